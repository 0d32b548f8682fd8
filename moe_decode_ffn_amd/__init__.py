"""MI355X (gfx950) decode-step MoE feed-forward layer with a gated shared expert.

``moe_decode_ffn_amd.ffn`` binds the HIP library (include/moe_ffn.h);
``moe_decode_ffn_amd.synth`` draws seeded synthetic layers and tokens;
``moe_decode_ffn_amd.build`` compiles the library for gfx950.
Importing the package loads nothing; the binding loads the library on first use.
"""
