"""Analytic decode cost model: FLOPs and HBM bytes per generated token.

Reproduction card, "What reproduces (and what does not)", claim C2: an exact
decode-FLOPs model gives a 54.5% FLOPs reduction of top-C sparse decoding
against full attention at the Qwen3-8B shape with a 32k context (the card
names the model's equations but does not print them).  "Key finding worth
flagging": at C = 2k the page-level baseline (Quest) attends the same number
of tokens and adds only its page-scan term 2*q*h*(T/P), a 1-4% FLOPs gap.

Readings taken (the plainest model consistent with those figures):
* FLOPs per generated token and decoder layer, a multiply-add counting 2:
  the linear layers, 2 * (hidden*Hq*D + 2*hidden*Hkv*D + Hq*D*hidden
  + 3*hidden*intermediate) (q, k, v and o projections, gated MLP), plus the
  attention, 4*Hq*D*N over the N attended tokens (q.k and the weighted V sum).
  N = T for full attention, min(C, T) for token-level sparse decoding.
  Embeddings, norms, rotary terms and the LM head are left out.
* The page-scan term: 2*D*Hq*(T/P) per layer (q = head_dim, h = query heads,
  P = page size), added to the sparse FLOPs.
* The selection itself (scoring every key with the predicted query,
  2*Hq*D*T, and the top-C select) runs off the decode path, on the selection
  stream; it is reported separately and not in the reduction.
With these readings the Qwen3-8B shape at T = 32768, C = 2048 gives exactly
6/11 = 54.5%, and the page-scan gap is 4.0% at P = 16 and 1.0% at P = 64.

HBM bytes per step of one layer (all B sequences), bf16 K/V: the decode path
reads the attended K and V rows, 2*Hkv*D*2 bytes per token attended; the
selection path scans K, Hkv*D*2 bytes per cached token.  hot_path_bytes is
the step-byte count of the score + select + attend path that the benchmark
reports.

The architecture hyperparameters below are the public Qwen3 model
configurations (hidden size, intermediate size), not figures from the pages;
the head counts, head_dim and layer counts are the workloads' own.

    python -m query_aware_sparse_amd.flops_model --model qwen3-8b --context 32768 --top-c 2048
"""
from __future__ import annotations

import argparse
import json
from dataclasses import dataclass
from typing import Dict, Iterable


@dataclass(frozen=True)
class Arch:
    name: str
    layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int


ARCHS = {
    "qwen3-8b": Arch("qwen3-8b", layers=36, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     intermediate=12288),
    "qwen3-32b": Arch("qwen3-32b", layers=64, hidden=5120, n_q_heads=64, n_kv_heads=8, head_dim=128,
                      intermediate=25600),
}


def linear_flops(a: Arch) -> int:
    """Projection and MLP FLOPs of one decoder layer for one token."""
    hq, hkv = a.n_q_heads * a.head_dim, a.n_kv_heads * a.head_dim
    return 2 * (a.hidden * hq + 2 * a.hidden * hkv + hq * a.hidden + 3 * a.hidden * a.intermediate)


def attention_flops(a: Arch, n_tokens: int) -> int:
    """q.k and the weighted V sum over n_tokens attended tokens, one layer, one token."""
    return 4 * a.n_q_heads * a.head_dim * n_tokens


def page_scan_flops(a: Arch, context: int, page: int) -> int:
    """Page-level selection's scan of the page summaries, one layer, one token."""
    return 2 * a.head_dim * a.n_q_heads * (context // page)


def decode_flops(a: Arch, context: int, top_c: int = 0, page: int = 0) -> Dict[str, int]:
    """Per generated token, all layers: full attention, token-level sparse
    (top_c tokens), and page-level sparse (top_c tokens plus the page scan)."""
    lin = linear_flops(a)
    c_eff = min(top_c, context)
    full = a.layers * (lin + attention_flops(a, context))
    sparse = a.layers * (lin + attention_flops(a, c_eff))
    out = {"full": full, "sparse": sparse,
           "selection_off_path": a.layers * 2 * a.n_q_heads * a.head_dim * context}
    if page:
        out["page_sparse"] = sparse + a.layers * page_scan_flops(a, context, page)
    return out


def reduction(a: Arch, context: int, top_c: int) -> float:
    """Fraction of decode FLOPs that token-level sparse decoding saves."""
    f = decode_flops(a, context, top_c)
    return 1.0 - f["sparse"] / f["full"]


def page_scan_gap(a: Arch, context: int, top_c: int, page: int) -> float:
    """Extra FLOPs of page-level over token-level sparse decoding, relative to the latter."""
    f = decode_flops(a, context, top_c, page)
    return f["page_sparse"] / f["sparse"] - 1.0


def kv_bytes(a: Arch, batch: int, context: int, top_c: int) -> Dict[str, int]:
    """HBM bytes of K/V per step of one layer (bf16): full attention, the sparse
    decode path (attended rows) and the selection path (the K scan)."""
    row = a.n_kv_heads * a.head_dim * 2
    c_eff = min(top_c, context)
    return {"full_attention": batch * 2 * row * context, "sparse_decode": batch * 2 * row * c_eff,
            "selection_scan": batch * row * context}


def hot_path_bytes(a: Arch, seq_lens: Iterable[int], top_c: int) -> int:
    """Step bytes of the score + select + attend path of one layer: per unit,
    the K scan T*D*2, the K and V gathers 2*C_eff*D*2, the index write and read
    8*C_eff, and the predicted query, actual query and output 3*G*D*4."""
    D, G = a.head_dim, a.n_q_heads // a.n_kv_heads
    total = 0
    for T in seq_lens:
        ce = min(top_c, T)
        total += a.n_kv_heads * (T * D * 2 + 2 * ce * D * 2 + 8 * ce + 3 * G * D * 4)
    return total


def main() -> int:
    ap = argparse.ArgumentParser(description="Analytic decode FLOPs and bytes (CPU).")
    ap.add_argument("--model", default="qwen3-8b", choices=sorted(ARCHS))
    ap.add_argument("--context", type=int, default=32768)
    ap.add_argument("--top-c", type=int, default=2048)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--page", type=int, nargs="*", default=[16, 64])
    args = ap.parse_args()
    a = ARCHS[args.model]
    f = decode_flops(a, args.context, args.top_c)
    print(json.dumps({
        "model": a.name, "context": args.context, "top_c": args.top_c,
        "decode_gflops_per_token": {k: v / 1e9 for k, v in f.items()},
        "flops_reduction_vs_full": reduction(a, args.context, args.top_c),
        "page_scan_gap": {str(p): page_scan_gap(a, args.context, args.top_c, p) for p in args.page},
        "kv_bytes_per_layer_step": kv_bytes(a, args.batch, args.context, args.top_c),
        "hot_path_bytes_per_layer_step": hot_path_bytes(a, [args.context] * args.batch, args.top_c),
    }, indent=1))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
