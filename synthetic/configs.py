"""The five workload shapes of the DiT block forward.

Each configuration is a model shape plus one packed batch.  A packed batch is a
list of segments.  A segment is one document: a contiguous run of tokens of one
modality, attended to only by itself, with its own position grid and one
modulation (conditioning) row.  Nothing here is derived; the derived tables
(cu_seqlens, per-token condition index, positions, cos/sin) are computed
independently by the oracle and by the library.

Shapes follow the workloads the pages describe:
  * tiny fp32 DiT: 2 blocks, hidden 128, 4 heads x 32, SwiGLU 512, RMSNorm,
    two packed documents of 64 and 96 tokens, RoPE split 8/12/12 over (t,h,w);
  * the music acoustic DiT (page "the 2.4B fp32 DiT onto the device", section
    "What moved, and onto what"): 24 blocks, hidden 2560, 20 heads x 128,
    partial rotary on 64 dims, LayerNorm, value*silu(gate) MLP with ffn 10240,
    128-channel 1x1 convolutions as GEMMs over 86 frames, 2 CFG branches;
  * the joint video+audio DiT (page "port the MiniMax-H3 omni-modal video+audio
    DiT", section "The device-resident forward"): hidden 6144, 48 heads x 128,
    SwiGLU 16384, RMSNorm, AdaLN indexed per token by modality, 3-axis RoPE on
    video tokens and 1-axis RoPE on audio tokens, at three batch shapes.
"""

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Modality:
    name: str
    io: str                      # 'none' | 'patch3d' | 'channel_major'
    channels: int                # latent channels C (0 when io == 'none')
    patch: Tuple[int, int, int]  # (pt, ph, pw) for 'patch3d'
    rope_axes: Tuple[int, ...]   # rotary sub-dimension per position axis; sums to rot_dim
    rope_grid: str = "integer"   # 'integer' positions | 'centered' cell centres of [-1, 1) times 2 pi

    @property
    def token_width(self) -> int:
        """Width of one token's latent vector entering the in-projection."""
        if self.io == "patch3d":
            return self.channels * self.patch[0] * self.patch[1] * self.patch[2]
        if self.io == "channel_major":
            return self.channels
        return 0


@dataclass(frozen=True)
class Segment:
    modality: int
    grid: Tuple[int, ...]        # token grid, one extent per rope axis of the modality
    cond_row: int

    @property
    def n_tokens(self) -> int:
        n = 1
        for g in self.grid:
            n *= g
        return n


@dataclass(frozen=True)
class CondRow:
    modality: int                # which per-modality AdaLN linear produces this row
    source: int                  # request index (timestep) or conditioning-vector index


@dataclass(frozen=True)
class DitConfig:
    name: str
    key_id: int                  # seeds the inputs of this configuration
    model_id: int                # seeds the weights (configurations of one model share weights)
    n_blocks: int
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    norm: str                    # 'rms' | 'layer'
    norm_eps: float
    mlp: str                     # 'gate_up' ([gate | up]) | 'value_gate' ([value | gate])
    rot_dim: int
    theta: float
    stream: str                  # 'f32' | 'bf16'
    cond_kind: str               # 'timestep' | 'vector'
    cond_dim: int
    modalities: Tuple[Modality, ...]
    segments: Tuple[Segment, ...]
    cond_rows: Tuple[CondRow, ...]
    n_requests: int
    io: bool                     # True: latents in, velocities out; False: tokens in, tokens out
    denoise_steps: int = 0
    shifts: Tuple[float, ...] = field(default_factory=tuple)
    cfg_replicate_latent: bool = False  # segment j + P reads the latent of segment j (P = half the segments)
    gemm: str = "stream"         # 'stream' | 'mxfp8' | 'mxfp4' (MXFP4 weights, MXFP8 activations): the four block GEMMs of a bf16 stream
    qkv_layout: str = "concat"   # 'concat' [q_all | k_all | v_all] | 'per_head' [q k v of head 0 | ...]
    qk_norm: bool = False        # per-head RMS norm of q and k (no weight) before RoPE

    @property
    def n_tokens(self) -> int:
        return sum(s.n_tokens for s in self.segments)

    @property
    def n_cond(self) -> int:
        return len(self.cond_rows)

    @property
    def n_mod(self) -> int:
        return len(self.modalities)


_VIDEO_6144 = Modality("video", "patch3d", 16, (1, 2, 2), (32, 48, 48))
_AUDIO_6144 = Modality("audio", "channel_major", 32, (1, 1, 1), (128,))
_VIDEO_6144_TOKENS = Modality("video", "none", 0, (1, 1, 1), (32, 48, 48))
_AUDIO_6144_TOKENS = Modality("audio", "none", 0, (1, 1, 1), (128,))

_WIDE = dict(hidden=6144, n_heads=48, head_dim=128, ffn=16384, norm="rms", norm_eps=1e-6,
             mlp="gate_up", rot_dim=128, theta=10000.0, stream="bf16", cond_kind="timestep",
             cond_dim=256)

C1 = DitConfig(
    name="c1_tiny_f32", key_id=1, model_id=1, n_blocks=2, hidden=128, n_heads=4, head_dim=32,
    ffn=512, norm="rms", norm_eps=1e-6, mlp="gate_up", rot_dim=32, theta=10000.0, stream="f32",
    cond_kind="timestep", cond_dim=128,
    modalities=(Modality("tokens", "none", 0, (1, 1, 1), (8, 12, 12)),),
    segments=(Segment(0, (4, 4, 4), 0), Segment(0, (4, 4, 6), 0)),
    cond_rows=(CondRow(0, 0),), n_requests=1, io=False)

C2 = DitConfig(
    name="c2_music_f32", key_id=2, model_id=2, n_blocks=24, hidden=2560, n_heads=20, head_dim=128,
    ffn=10240, norm="layer", norm_eps=1e-6, mlp="value_gate", rot_dim=64, theta=10000.0,
    stream="f32", cond_kind="vector", cond_dim=256,
    modalities=(Modality("music", "channel_major", 128, (1, 1, 1), (64,)),),
    segments=(Segment(0, (86,), 0), Segment(0, (86,), 1)),
    cond_rows=(CondRow(0, 0), CondRow(0, 1)), n_requests=2, io=True, cfg_replicate_latent=True,
    denoise_steps=30, shifts=(1.0,))

C3 = DitConfig(
    name="c3_block_bf16", key_id=3, model_id=3, n_blocks=1, **_WIDE,
    modalities=(_VIDEO_6144_TOKENS, _AUDIO_6144_TOKENS),
    segments=(Segment(0, (8, 48, 64), 0), Segment(1, (2048,), 1)),
    cond_rows=(CondRow(0, 0), CondRow(1, 0)), n_requests=1, io=False)

C4 = DitConfig(
    name="c4_full_bf16", key_id=4, model_id=4, n_blocks=64, **_WIDE,
    modalities=(_VIDEO_6144, _AUDIO_6144),
    segments=(Segment(0, (4, 32, 64), 0), Segment(1, (1024,), 1),
              Segment(0, (4, 32, 64), 2), Segment(1, (1024,), 3)),
    cond_rows=(CondRow(0, 0), CondRow(1, 0), CondRow(0, 1), CondRow(1, 1)), n_requests=2, io=True)

C5 = DitConfig(
    name="c5_denoise_bf16", key_id=5, model_id=4, n_blocks=64, **_WIDE,
    modalities=(_VIDEO_6144, _AUDIO_6144),
    segments=(Segment(0, (8, 32, 64), 0), Segment(1, (2048,), 1)),
    cond_rows=(CondRow(0, 0), CondRow(1, 0)), n_requests=1, io=True,
    denoise_steps=50, shifts=(12.0, 3.0))

# The 64-block model with its four block GEMMs on MXFP8 operands (the low-precision arm).
C3_MX = replace(C3, name="c3_block_mxfp8", gemm="mxfp8")
C4_MX = replace(C4, name="c4_full_mxfp8", gemm="mxfp8")
C3_MX4 = replace(C3, name="c3_block_mxfp4", gemm="mxfp4")
C4_MX4 = replace(C4, name="c4_full_mxfp4", gemm="mxfp4")

# The video VAE decoder's ViT block at the pages' width (32 heads x 64, rotary
# on 0.75 of each head split over 3 axes, theta 100, fp32): per-head qkv rows,
# per-head q/k norm, centred coordinates.  The MLP width is a reading (4x).
VIT = DitConfig(
    name="vit3d_block_f32", key_id=6, model_id=6, n_blocks=1, hidden=2048, n_heads=32, head_dim=64, ffn=8192,
    norm="rms", norm_eps=1e-6, mlp="gate_up", rot_dim=48, theta=100.0, stream="f32", cond_kind="vector",
    cond_dim=4, modalities=(Modality("video", "none", 0, (1, 1, 1), (16, 16, 16), "centered"),),
    segments=(Segment(0, (2, 8, 12), 0), Segment(0, (1, 4, 6), 0)),
    cond_rows=(CondRow(0, 0),), n_requests=1, io=False, qkv_layout="per_head", qk_norm=True)

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5, C3_MX, C4_MX, VIT)}
_SHORT = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5, "c3_mxfp8": C3_MX, "c4_mxfp8": C4_MX,
          "c3_mxfp4": C3_MX4, "c4_mxfp4": C4_MX4, "vit": VIT}


def get_config(name: str) -> DitConfig:
    if name in _SHORT:
        return _SHORT[name]
    return CONFIGS[name]


def scaled(cfg: DitConfig, **changes) -> DitConfig:
    """A copy of ``cfg`` with some fields replaced (smaller test shapes)."""
    from dataclasses import replace
    return replace(cfg, **changes)
