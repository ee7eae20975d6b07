"""CPU oracle for the rolling-window KV streaming-decode path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
statement of what the GPU path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product library (``rolling_window_kv_amd``) never does, and the
two share no code, tables or constants.  Inputs are passed in as arrays (the
seeded generators live in ``rolling_window_kv_amd.synth``, which holds no
arithmetic of the method).

Sources (the web pages this follows; cited by title and section):

* "Audio8 ASR Infinite 无限长转写原理: Rolling KV Cache 如何让内存与延迟保持恒定"
  (m.lsln.cn news 158448) -- sections "Rolling KV Cache 三步拆解" (fixed 30 s
  window, exact RoPE re-basing, constant per-step cost) and "三档音频时钟".
* "Edge0/Audio8-ASR-Infinite · Hugging Face" (Chinese mirror of the model
  card) -- "优化操作点", "架构" / checkpoint specification, "使用 vLLM 进行全天候推理".
* "Edge0-AI / Audio8-ASR-Infinite" (README mirror) -- "Optimized operation points".
* The voxtral.c rolling-KV-cache explainer (kwkr.cn news 561915) -- sections
  一 (window table), 二 (compaction in three steps, logical position),
  三 (encoder incremental window), 四 (continuous mode).

Modules
-------
``bf16``      round-to-nearest-even to bfloat16 from float64 (own implementation)
``rope``      rotary angles and the exact rotation R(p)
``schedule``  per-step integer plans: ring re-base mode, compaction mode,
              encoder chunk ring
``attention`` exact attention over the window at absolute / logical positions
``storage``   storage-faithful simulation: bf16 rounding at every point the
              method stores K (append, each re-base, compensated hi/lo)
``pages``     the constants the pages print, and the derived window sizes
"""
