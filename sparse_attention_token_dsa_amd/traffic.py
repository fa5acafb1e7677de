"""Measured HBM traffic of the decode scan and the fused prefill, from
rocprofv3 counters.

Two counter runs of the same program, then a summary:

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o p -- \
      python3 -m sparse_attention_token_dsa_amd.traffic run
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o p -- \
      python3 -m sparse_attention_token_dsa_amd.traffic run
  python3 -m sparse_attention_token_dsa_amd.traffic summarize OUT

`run` launches the DSA decode selector on the L = 131072, batch-8, 64-head
workload a few times, then the same selector on the keys quantized to E4M3,
the fused prefill (T = 4096 over 28672 cached keys,
k = 2048) twice, then a plain copy kernel (torch's elementwise add of a zero
into a second 256 MiB fp32 tensor: 256 MiB read, 256 MiB written).
`summarize` reads both runs, calibrates each counter on the copy kernel
(counter bytes / known bytes) and writes, per launch of each measured kernel,
the HBM bytes fetched and written divided by those factors to traffic.json
(keyed by a digest of the kernel's sources, which bench.py checks before it
reports the figure).

MFMA utilisation of the fused prefill, one more counter run:

  rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES \
      SQ_INSTS_VALU SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE \
      GRBM_GUI_ACTIVE --output-format csv -d OUT/mfma -o p -- \
      python3 -m sparse_attention_token_dsa_amd.traffic run_prefill [fp8q]
  python3 -m sparse_attention_token_dsa_amd.traffic summarize_mfma OUT [fp8q]

(fp8q: the same prefill on the FP8 key cache with the query in E4M3, stored
under "prefill_fused_fp8q_mfma".)

`summarize_mfma` stores, per prefill launch (median over the launches): the
raw counters, MFMA-busy cycles per SIMD over the GPU's active cycles, VALU
instructions per MFMA instruction and LDS bank-conflict cycles over LDS-active
cycles, under "prefill_fused_mfma" in traffic.json.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "traffic.json")
SCAN_SOURCES = ["scan.hip", "sa_frag.h", "sa_common.h"]
SCAN_KERNEL = "scan_kernel<4, 4, 1, 4, 64, true, false, false>"
SCAN_POOL_KERNEL = "scan_kernel<4, 4, 1, 4, 32, true, false, true>"
SCAN_ROUTED_KERNEL = "scan_kernel<1, 4, 1, 4, 64, true, true, false>"
SCAN8_KERNEL = "scan8_kernel<4, true, false>"
SCAN8Q_KERNEL = "scan8_kernel<4, true, true>"
SCAN8_SOURCES = ["scan8.hip", "sa_frag.h", "sa_common.h"]
PREFILL_SOURCES = ["prefill.hip", "sa_frag.h", "sa_common.h"]
PREFILL_KERNEL = "prefill_kernel<4, false, false>"
PREFILL8_KERNEL = "prefill_kernel<4, true, false>"
COPY_BYTES = 256 << 20
COPY_KERNEL = "CUDAFunctorOnSelf_add<float>"  # torch.add(src, 0.0, out=dst)


def source_digest(names=SCAN_SOURCES):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(HERE, "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def run():
    import numpy as np
    import torch

    from sparse_attention_token_dsa_amd import api, synth

    dev = torch.device("cuda:0")
    p = synth.make_config("misa_128k_h64")
    q = torch.from_numpy(p["q"].view(np.int16)).to(dev)
    w = torch.from_numpy(p["w"]).to(dev)
    K = torch.from_numpy(p["K"].view(np.int16)).to(dev)
    for _ in range(4):
        api.indexer_score_topk(q, w, K, p["offset"], 2048)
    reps_b = torch.empty((8, 1024, 2, 128), dtype=torch.int16, device=dev)
    reps_B = torch.empty((8, 128, 2, 128), dtype=torch.int16, device=dev)
    for _ in range(4):
        api.indexer_score_topk_pooled(q, w, K, p["offset"], 2048, 128, 1024, out_small=reps_b,
                                      out_large=reps_B)
    for _ in range(4):
        api.misa_route(q, w, K, p["offset"], 2048, 1024, 8, 0, pooled=reps_B, want_heads=False)
    torch.cuda.synchronize()
    codes, scales = api.quantize_keys_fp8(K)
    for _ in range(4):
        api.indexer_score_topk_fp8(q, w, codes, scales, p["offset"], 2048)
    for _ in range(4):
        api.indexer_score_topk_fp8q(q, w, codes, scales, p["offset"], 2048)
    torch.cuda.synchronize()
    del codes, scales
    pp = synth.make_config("prefill_chunked")
    q = torch.from_numpy(pp["q"].view(np.int16)).to(dev)
    w = torch.from_numpy(pp["w"]).to(dev)
    K = torch.from_numpy(pp["K"].view(np.int16)).to(dev)
    for _ in range(2):
        api.indexer_score_topk(q, w, K, pp["offset"], 2048)
    codes, scales = api.quantize_keys_fp8(K)
    for _ in range(2):
        api.indexer_score_topk_fp8q(q, w, codes, scales, pp["offset"], 2048)
    torch.cuda.synchronize()
    del codes, scales
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    print("traffic run done", flush=True)


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU",
                 "SQ_INSTS_MFMA", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4   # compute units x SIMDs
XCDS = 8


def run_prefill(launches=6, fp8q=False):
    """The fused prefill at T = 4096 over 28672 cached keys, k = 2048 (fp8q:
    on the FP8 key cache with the query in E4M3)."""
    import numpy as np
    import torch

    from sparse_attention_token_dsa_amd import api, synth

    dev = torch.device("cuda:0")
    pp = synth.make_config("prefill_chunked")
    q = torch.from_numpy(pp["q"].view(np.int16)).to(dev)
    w = torch.from_numpy(pp["w"]).to(dev)
    K = torch.from_numpy(pp["K"].view(np.int16)).to(dev)
    oi = torch.empty((1, pp["T"], 2048), dtype=torch.int32, device=dev)
    if fp8q:
        codes, scales = api.quantize_keys_fp8(K)
        for _ in range(launches):
            api.indexer_score_topk_fp8q(q, w, codes, scales, pp["offset"], 2048, out_idx=oi)
    else:
        for _ in range(launches):
            api.indexer_score_topk(q, w, K, pp["offset"], 2048, out_idx=oi)
    torch.cuda.synchronize()
    print("prefill counter run done", flush=True)


def summarize_mfma(out_dir, fp8q=False):
    vals = {c: _per_dispatch(os.path.join(out_dir, "mfma"), c) for c in MFMA_COUNTERS}
    raw = {c: _pick(v, PREFILL8_KERNEL if fp8q else PREFILL_KERNEL) for c, v in vals.items()}
    gui = raw["GRBM_GUI_ACTIVE"] / XCDS          # the counter sums the XCDs
    rec = {
        "kernel": "prefill_fused_fp8q" if fp8q else "prefill_fused",
        "source_digest": source_digest(PREFILL_SOURCES),
        "counters_median_per_launch": raw,
        "active_cycles": gui,
        "mfma_busy_per_simd": raw["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS,
        "mfma_busy_frac": raw["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / gui,
        "valu_per_mfma": raw["SQ_INSTS_VALU"] / raw["SQ_INSTS_MFMA"],
        "lds_bank_conflict_frac": raw["SQ_LDS_BANK_CONFLICT"] / raw["SQ_LDS_IDX_ACTIVE"],
    }
    try:
        with open(TRAFFIC_FILE) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec["prefill_fused_fp8q_mfma" if fp8q else "prefill_fused_mfma"] = rec
    print(json.dumps(rec, indent=1))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
        f.write("\n")


def _per_dispatch(run_dir, counter):
    """{kernel name: [counter value per dispatch]} from one --pmc run."""
    out = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(d, needle):
    hits = [v for k, v in d.items() if needle in k]
    if not hits:
        raise SystemExit("no dispatch of %r in the counter run" % needle)
    return statistics.median(hits[0])


def summarize(out_dir):
    fetch = _per_dispatch(os.path.join(out_dir, "fetch"), "FETCH_SIZE")
    write = _per_dispatch(os.path.join(out_dir, "write"), "WRITE_SIZE")
    copy_f, copy_w = _pick(fetch, COPY_KERNEL), _pick(write, COPY_KERNEL)
    f_fetch = copy_f * 1024.0 / COPY_BYTES
    f_write = copy_w * 1024.0 / COPY_BYTES
    try:
        with open(TRAFFIC_FILE) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    for name, needle, sources in (("scan_dsa", SCAN_KERNEL, SCAN_SOURCES),
                                  ("scan_dsa_pool", SCAN_POOL_KERNEL, SCAN_SOURCES),
                                  ("scan_routed", SCAN_ROUTED_KERNEL, SCAN_SOURCES),
                                  ("scan_dsa_fp8", SCAN8_KERNEL, SCAN8_SOURCES),
                                  ("scan_dsa_fp8q", SCAN8Q_KERNEL, SCAN8_SOURCES),
                                  ("prefill_fused", PREFILL_KERNEL, PREFILL_SOURCES),
                                  ("prefill_fused_fp8q", PREFILL8_KERNEL, PREFILL_SOURCES)):
        kf, kw = _pick(fetch, needle), _pick(write, needle)
        rec = {
            "kernel": name,
            "source_digest": source_digest(sources),
            "fetch_kib_per_launch": kf,
            "write_kib_per_launch": kw,
            "copy_kernel_bytes_each_way": COPY_BYTES,
            "copy_fetch_kib": copy_f,
            "copy_write_kib": copy_w,
            "factor_fetch": f_fetch,
            "factor_write": f_write,
            "bytes_per_launch": kf * 1024.0 / f_fetch + kw * 1024.0 / f_write,
        }
        allrec[name] = rec
        print(json.dumps(rec, indent=1))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) >= 2 and sys.argv[1] == "run_prefill":
        run_prefill(fp8q=len(sys.argv) >= 3 and sys.argv[2] == "fp8q")
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize_mfma":
        summarize_mfma(sys.argv[2], fp8q=len(sys.argv) >= 4 and sys.argv[3] == "fp8q")
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize":
        summarize(sys.argv[2])
    else:
        raise SystemExit(__doc__)
