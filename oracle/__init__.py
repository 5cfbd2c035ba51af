"""fp64 CPU oracle for the sink-GQA attention path -- TEST INFRASTRUCTURE.

Plain, slow, obviously correct numpy code that states what the path computes,
so the HIP kernels can be checked against it element by element.  It is not
part of the product: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in here.  It
shares no code with the HIP library (no kernels, headers, helpers, tables or
constants) and imports nothing from it.

Modules
  rounding   fp64 -> bf16 / fp32 rounding of results (direct, ties to even)
  yarn       base RoPE schedule, NTK-by-parts rotations, YaRN blend,
             concentration, rotation of Q/K at global positions
  attention  masks, sink-augmented softmax, GQA; a per-query form and a
             dense mask-matrix form
  kvcache    append-only cache with snapshot/restore; KV byte count
  qkv        fused qkv projection (x W^T + b rounded once) and its [Q | K | V] split
  moe        top-k router with a stable tie-break, softmax over the selected
             logits, dispatch by expert, SwiGLU experts, weighted combine
  ring       sliding-window ring cache of band layers (W rows, slot p mod W),
             its band mask in ring coordinates, KV entry counts
  sampling   logit bias and penalties, temperature, top-k / top-p / min-p,
             greedy decode and the draw from a given uniform

Sources are cited as page title + section.  The pages:
  "MoE-Xtend" README (sections DESIGN CONTRACTS, ARCHITECTURE,
      TOKEN STREAM (DECODE), ATTENTION STACK, ROPE + SCALING, KV CACHE,
      NOTATION, SAMPLING CONTROLS)
  "GQA Attention" study note on gpt-oss (section "How it works")
  "MoE-Xtend" project summary page
  "GPT-OSS-Lite" README (shapes; the KV-cache reduction figures) and visual
      guide (shapes; the KV-cache calculator)

Every function here is pinned by the ``-m "not gpu"`` tests against closed
forms, special cases that reduce to library routines, brute force on tiny
inputs, or numbers the pages print; none is marked "parity unpinned".
"""
