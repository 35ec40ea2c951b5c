"""MI355X-native (gfx950) FLUX.2-klein / FLUX.3-Klein denoising-transformer forward pass."""
