"""MI355X (gfx950) online-softmax kernels behind a C ABI; see include/tea.h."""
