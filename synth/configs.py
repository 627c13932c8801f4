"""The five synthetic workloads (sizes, precisions, stream counts, step counts).

Model sizes follow the Parakeet-EOU-120M model card ("Config" table: 17 encoder layers,
hidden 512, attention context 70) and the fluidaudio-web streaming spec ("Why this is
provably correct": chunk 2, left 70; "State": 14-frame mel tail, 8-column conv cache;
"Status", Nemotron variant: right context 3 with a provisional tail).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class EncConfig:
    name: str
    seed: int               # master seed of this workload
    n_layers: int = 17
    d_model: int = 512
    n_heads: int = 8
    d_ff: int = 2048
    dw_kernel: int = 9      # depthwise kernel; the conv cache holds dw_kernel-1 columns
    att_left: int = 70      # Lc: left attention context, also the K/V cache depth
    att_chunk: int = 2      # frames per attention chunk (push granularity)
    att_right: int = 0      # right context (lookahead variant only)
    n_emit: int = 2         # frames emitted per stream per push
    n_lookahead: int = 0    # provisional frames recomputed every pass (lookahead variant)
    joint_dim: int = 640    # 0 = no joint projection
    frontend: int = 0       # 1: 3 causal stride-2 convs over log-mel; 2: the 2-D time x frequency stack
    fe_channels: int = 256  # channels of the 2-D stack
    mel_bins: int = 128
    mel_per_chunk: int = 16
    mel_tail: int = 14
    dtype: str = "f32"      # "f32", "bf16" or "i8w" (float32 with int8 dense weights)
    streams: int = 1
    chunks: int = 100       # pushes per stream in the workload
    staggered: bool = False  # streams start from injected random states
    token_classes: int = 1026  # check-only token head: 1024 vocab + blank + EOU

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    @property
    def n_compute(self) -> int:
        """Frames run through the layers per stream per push."""
        return self.n_emit + self.n_lookahead

    @property
    def conv_cache(self) -> int:
        return self.dw_kernel - 1

    def replace(self, **kw) -> "EncConfig":
        return dataclasses.replace(self, **kw)


C1 = EncConfig(name="C1_tiny_f32", seed=0, n_layers=2, d_model=64, n_heads=4, d_ff=256,
               joint_dim=0, dtype="f32", streams=1, chunks=100)
C2 = EncConfig(name="C2_eou_f32_1stream", seed=1, dtype="f32", streams=1, chunks=1000)
C3 = EncConfig(name="C3_eou_bf16_256streams", seed=2, dtype="bf16", streams=256, chunks=200,
               staggered=True)
C4 = EncConfig(name="C4_eou_bf16_1024streams_frontend", seed=3, dtype="bf16", streams=1024,
               chunks=100, staggered=True, frontend=True)
C5 = EncConfig(name="C5_lookahead_bf16_512streams", seed=4, dtype="bf16", streams=512, chunks=300,
               staggered=True, att_right=3, n_emit=2, n_lookahead=8)

# the 1024-stream front-end workload with the 2-D time x frequency subsampling stack
C4S = C4.replace(name="C4S_eou_bf16_1024streams_frontend2d", frontend=2)

# the one-stream encoder of C2 (same seed: same weights and inputs) with int8 dense weights
C2Q = C2.replace(name="C2_eou_i8w_1stream", dtype="i8w")

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5, "C2Q": C2Q, "C4S": C4S}


@dataclass(frozen=True)
class DecConfig:
    """Greedy RNNT + EOU decoding after the encoder: predictor (embedding + LSTM stack, its
    output projected to the joint width) and the joint after projection over vocab + blank +
    EOU classes, fed the encoder's projected frames."""
    name: str
    seed: int
    joint_dim: int = 640        # P: width of the projected encoder and predictor outputs
    pred_hidden: int = 640      # H: embedding and LSTM width
    pred_layers: int = 2
    vocab: int = 1024           # V; blank = V, EOU = V + 1
    max_symbols: int = 4        # emissions per frame before the decoder moves on
    blank_bias: float = 2.5     # added to the blank class's joint bias (synthetic weights)
    streams: int = 1
    frames: int = 2             # frames per decode call (one encoder chunk)
    calls: int = 1000

    @property
    def classes(self) -> int:
        return self.vocab + 2

    def replace(self, **kw) -> "DecConfig":
        return dataclasses.replace(self, **kw)


D1 = DecConfig(name="D1_greedy_1stream", seed=11, streams=1, calls=1000)
D2 = DecConfig(name="D2_greedy_1024streams", seed=12, streams=1024, calls=100)
DEC_CONFIGS = {"D1": D1, "D2": D2}


@dataclass(frozen=True)
class BeamConfig:
    """Batched MALSD beam search over whole utterances of projected encoder frames, with the
    greedy decoder's prediction network and joint (same parameter names and shapes)."""
    name: str
    seed: int
    joint_dim: int = 640
    pred_hidden: int = 640
    pred_layers: int = 2
    vocab: int = 1024
    beam: int = 8
    max_symbols: int = 10       # the beam decoder's default label cap
    blank_bias: float = 3.0     # added to the blank class's joint bias (synthetic weights)
    silence: float = 0.5        # fraction of frames pushed towards blank
    silence_gain: float = 4.0   # strength of that push
    score_norm: bool = True
    streams: int = 64
    frames: int = 188           # 15 s at 80 ms per encoder frame
    min_frames: int = 94        # utterance lengths uniform in [min_frames, frames]

    @property
    def classes(self) -> int:
        return self.vocab + 2

    def replace(self, **kw) -> "BeamConfig":
        return dataclasses.replace(self, **kw)


B8 = BeamConfig(name="B8_malsd_beam8_64utt", seed=21)
# short utterances of the same model shape, for parity at many beam widths
B8S = B8.replace(name="B8S_malsd_short", seed=22, frames=24, min_frames=1, streams=48)
BEAM_CONFIGS = {"B8": B8, "B8S": B8S}


def get_config(key: str) -> EncConfig:
    return CONFIGS[key]


@dataclass(frozen=True)
class MelConfig:
    """Streaming log-mel front: raw 16 kHz audio chunks of ``hops`` 10 ms hops per stream."""
    name: str
    seed: int
    sample_rate: int = 16000
    n_fft: int = 512
    win_length: int = 400
    hop: int = 160
    n_mels: int = 128
    fmin: float = 0.0
    fmax: float = 8000.0
    preemph: float = 0.97
    out_dtype: str = "f32"
    streams: int = 1
    hops: int = 16          # one encoder chunk: 16 mel frames = 160 ms
    chunks: int = 100

    def replace(self, **kw) -> "MelConfig":
        return dataclasses.replace(self, **kw)


A4 = MelConfig(name="A4_logmel_1024streams", seed=5, streams=1024, chunks=100, out_dtype="bf16")
MEL_CONFIGS = {"A4": A4}