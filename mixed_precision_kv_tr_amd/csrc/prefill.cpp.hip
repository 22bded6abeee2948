// Prefill routed attention (placeholder until the MFMA kernel lands).
#include "common.h"

tr_status tr_prefill_launch(tr_kv_cache* c, int layer, int p0, const uint16_t* q, const uint8_t* mode, int T,
                            int window, uint16_t* out, hipStream_t stream) {
  (void)c; (void)layer; (void)p0; (void)q; (void)mode; (void)T; (void)window; (void)out; (void)stream;
  return TR_ERR_UNSUPPORTED;
}
