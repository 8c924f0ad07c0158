"""bench.py's host-side arithmetic: the algorithmic bytes it divides by the measured time, and
its refusal of more than one GPU.  No GPU is used."""
import bench
from long_context_decode_flash_amd import workloads as W


def test_token_bytes():
    # K codes + K scale + V codes + one fp16 scale per 32 dims
    assert bench.token_bytes(256, 4) == 256 + 2 + 128 + 16 == 402
    assert bench.token_bytes(64, 4) == 64 + 2 + 32 + 4 == 102
    assert bench.token_bytes(256, 8) == 256 + 2 + 256 + 16


def test_headline_bytes():
    wl = W.WORKLOADS["ctx184k_c2"]
    lens = [wl.seq_len] * wl.n_seq
    kv = 2 * 92160 * 4 * 402
    assert kv == 296_386_560  # the KV bytes of the 184K-token pool
    q = 2 * 1 * 24 * 256 * 2
    pt = 2 * 1440 * 4
    out = 2 * 1 * 24 * 257 * 4
    assert bench.decode_algorithmic_bytes(wl, lens) == kv + q + pt + out


def test_window_bytes():
    wl = W.WORKLOADS["ctx184k_c2"]
    lens = [wl.seq_len] * wl.n_seq
    w = 65536
    # each sequence: its last 65,536 tokens (one row), pages 409 .. 1439 of 64 tokens
    t0 = 92160 - 65536
    kv = 2 * w * 4 * 402
    pt = 2 * ((92160 - 1) // 64 - t0 // 64 + 1) * 4
    q, out = 2 * 24 * 256 * 2, 2 * 24 * 257 * 4
    assert bench.decode_algorithmic_bytes(wl, lens, 4, w) == kv + q + pt + out
    # a window longer than the context is the whole context
    assert bench.decode_algorithmic_bytes(wl, lens, 4, 10 ** 6) == \
        bench.decode_algorithmic_bytes(wl, lens)
    # MTP rows: the first row's window starts n_rows - 1 tokens earlier
    assert bench.attended_range(262144, 4, 1000) == (262144 - 4 - 1000 + 1, 262144)


def test_prefill_flops():
    # position i of a chunk of C at the end of L tokens attends L - C + i + 1 tokens; 4D flops
    # per token per query head (2D for Q K^T, 2D for P V)
    assert bench.prefill_attn_flops([5], 3, 1, 64) == (3 + 4 + 5) * 4 * 64
    # a chunk longer than the context: positions below zero see nothing
    assert bench.prefill_attn_flops([2], 4, 1, 64) == (1 + 2) * 4 * 64
    # the last 1,024-position chunk of both 92,160-token sequences, 24 query heads, D = 256
    per_seq = 1024 * (92160 - 1024) + 1024 * 1025 // 2
    assert bench.prefill_attn_flops([92160, 92160], 1024, 24, 256) == 2 * per_seq * 24 * 1024


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
