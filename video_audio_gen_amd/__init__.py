"""MI355X (gfx950) diffusion-transformer block forward: a C-ABI HIP library
(``libdit.so``, declared in ``include/dit.h``) and its thin Python binding
(``video_audio_gen_amd.dit``)."""

__all__ = ["dit"]
