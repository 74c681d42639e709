"""Row-wise softmax cross-entropy on MI355X (gfx950)."""
