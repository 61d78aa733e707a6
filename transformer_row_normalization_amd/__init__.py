"""transformer_row_normalization_amd: fused last-axis row normalization
(RMSNorm, LayerNorm, dual-output q/k head RMSNorm) for MI355X (gfx950)."""
