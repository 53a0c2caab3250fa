"""MI355X-native pooled block-sparse attention for diffusion-LLM denoising."""
