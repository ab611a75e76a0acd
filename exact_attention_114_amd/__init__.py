"""MI355X-native exact attention (FlashAttention forward) for gfx950."""
