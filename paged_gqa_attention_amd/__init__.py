"""libpagedattn: paged GQA decode attention for MI355X (gfx950).

``paged_gqa_attention_amd.pagedattn`` is the Python binding of the C ABI in
``include/pagedattn.h``; importing it loads the built HIP library and raises if
it is missing. ``paged_gqa_attention_amd.build`` compiles that library.
"""
