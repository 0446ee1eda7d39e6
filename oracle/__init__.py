"""CPU oracle for decode attention over a bounded KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's cpu_baseline leg use it.  It shares no code with the HIP path
(it imports only the `synth` input generators and numpy).

It is a plain, slow, float64 statement of what the decode step computes,
written from the pages' definitions:

  ring        which positions a sink + window cache holds (closed form) and
              the slot each position occupies; a literal ring simulation and
              the concat-and-prune manager, for pinning.
  rope        rotary position embedding at an absolute position.
  rounding    float64 -> bf16 / float32 rounding (nearest, ties to even).
  attention   softmax attention of one query over an explicit set of rows.
  decode      expected outputs of the workloads, from the full synthetic
              history, never from a slot or a block table.
  kvbytes     the pages' KV byte formulas.

Pages are cited by address and section:
  [ring]   http://www.2kiu.com/news/4318096/        (sliding window + ring KV buffer)
  [share]  http://www.pwwt.cn/news/6215824/         (KV sharing, block tables, GQA)
  [sink]   https://openeuler.csdn.net/6ad3842349ed150a32d85530.html (attention sinks)
  [kvc]    http://www.pwwt.cn/news/5010196/         (KV cache fundamentals)
  [pool]   https://www.cloudlnk.cn/blog/kv-cache-paging (fixed KV pool, slot mask)

Parity status of each function is stated in its module.  Not fixed by the
pages: the RoPE pairing convention and frequencies (rope.py pins both
against two library implementations of the rotary embedding instead), and
the exact ring slot chosen for a position (ring.slot_of; the set of
positions held is pinned, the slot index is a reading).
"""
