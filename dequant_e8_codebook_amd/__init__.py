"""MI355X (gfx950) E8-lattice-codebook linear layer: C-ABI library libglq.so
(include/glq.h) and its thin Python binding (dequant_e8_codebook_amd.glq)."""
