// Routing selection (sigmoid + bias keys, sorted top-k, renormalised weights,
// validity mask), shared by moe_route's projection and logits-in modes.
#pragma once

#include <stdint.h>

namespace moe {

// Per token t: logits[t,e] = scale * sum_p partials[p][t][e] (written to
// `logits`), or read from `logits` when logits_in != 0 (partials unused);
// then ids/weights as moe_route defines them. With `hist` set (zeroed
// beforehand), every valid pick j of token t also adds one to
// hist[(t k + j) / hist_tile][id]: the per-tile expert histograms of
// moe_dispatch's slots. Returns a moe_status.
int run_select(const float* partials, int nsplit, float scale, int logits_in, const float* bias,
               const uint8_t* mask, int T, int E, int k, float* logits, int32_t* ids, float* w,
               int32_t* hist, int hist_tile, void* stream);

}  // namespace moe
