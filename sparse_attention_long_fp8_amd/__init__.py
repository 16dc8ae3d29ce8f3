"""libdsa: DeepSeek Sparse Attention hot path for MI355X (gfx950).

The HIP library is loaded on first use by :mod:`.binding`; importing the
package (e.g. for the input generator) does not need a GPU.
"""
