// Continuous-mode restart policy (host code only; no device work).
//
// voxtral.c rolling-KV explainer, section 四: in live transcription the
// runtime restarts the decoder hard (no decoder context kept; the encoder
// cache and the streaming pipeline continue) when the model ends an
// utterance (EOS), when the decoder cache would grow past
// STREAM_MAX_DECODE_KV positions (bounding the attention cost), on a run of
// control tokens (a decoder looping on them), and when audio advances while
// the decoder produces nothing (watchdog).  Per stream and clock step the
// caller reports the token the decoder emitted (a text token, a control
// token, or none) and restarts the streams this returns with
// rkv_reset_streams.

#include "rkv.h"

extern "C" int rkv_restart_step(const rkv_restart_cfg* cfg, rkv_restart_state* h_state,
                                int32_t num_streams, const int32_t* h_token, int32_t* h_reason,
                                int32_t* h_restart) {
  if (!cfg || !h_state || !h_token || num_streams < 1) return RKV_EINVAL;
  if (cfg->text_token_min < 0) return RKV_EINVAL;
  int32_t count = 0;
  for (int32_t s = 0; s < num_streams; ++s) {
    rkv_restart_state& c = h_state[s];
    const int32_t tok = h_token[s];
    // one decoder position per step; the runs of control tokens and of
    // steps without a token
    c.decode_len += 1;
    const bool control = tok >= 0 && tok < cfg->text_token_min;
    c.nontext = control ? c.nontext + 1 : 0;
    c.idle = tok < 0 ? c.idle + 1 : 0;
    // the conditions in the page's order; the first that holds is reported
    int32_t reason = RKV_RESTART_NONE;
    if (cfg->eos_token >= 0 && tok == cfg->eos_token)
      reason = RKV_RESTART_EOS;
    else if (cfg->max_decode_kv > 0 && c.decode_len >= cfg->max_decode_kv)
      reason = RKV_RESTART_KV_OVERFLOW;
    else if (cfg->nontext_run > 0 && c.nontext >= cfg->nontext_run)
      reason = RKV_RESTART_NONTEXT_RUN;
    else if (cfg->stall_steps > 0 && c.idle >= cfg->stall_steps)
      reason = RKV_RESTART_STALL;
    if (reason != RKV_RESTART_NONE) {
      c.decode_len = 0;
      c.nontext = 0;
      c.idle = 0;
      c.restarts += 1;
      if (h_restart) h_restart[count] = s;
      ++count;
    }
    if (h_reason) h_reason[s] = reason;
  }
  return count;
}
