// Table of argument cases for the host-side checks of every libhs2 entry
// point (kv_cache_reuse_hs2_amd/csrc/validate.cpp), built on its own with the
// address and undefined-behaviour sanitizers by test_host_checks.py.  Device
// pointers are stand-in addresses that are never dereferenced; a case passes
// when the check returns the expected status.  Prints one line per mismatch
// and the totals; exits 1 on any mismatch.
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "validate.h"

using namespace hs2;

namespace {

int g_cases = 0, g_bad = 0;

void expect(const char* name, hs2_status got, hs2_status want) {
  ++g_cases;
  if (got != want) {
    ++g_bad;
    printf("MISMATCH %s: got %d, want %d\n", name, (int)got, (int)want);
  }
}

// Aligned and misaligned stand-in addresses (never dereferenced).
template <typename T>
const T* at(uintptr_t a) { return reinterpret_cast<const T*>(a); }
const uintptr_t A = 0x100000, M = 0x100008;

hs2_attn_desc decode_desc() {
  hs2_attn_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 4; d.n_q = 1; d.n_heads = 32; d.head_dim = 128; d.tile_q = 1;
  d.k_top = 1024; d.window = 128; d.causal = 1; d.sm_scale = 0.08838834764831845f;
  d.dtype = HS2_BF16; d.k_scale = 1.f; d.v_scale = 1.f;
  return d;
}

hs2_attn_desc prefill_desc() {
  hs2_attn_desc d = decode_desc();
  d.batch = 1; d.n_q = 8192; d.tile_q = 64;
  return d;
}

void set_dtype(hs2_attn_desc* d, int v) { memcpy(&d->dtype, &v, sizeof v); }

void desc_cases() {
  const hs2_attn_desc base = decode_desc();
  expect("desc null", check_desc(nullptr), HS2_EINVAL);
  expect("desc decode ok", check_desc(&base), HS2_OK);
  const hs2_attn_desc pf = prefill_desc();
  expect("desc prefill ok", check_desc(&pf), HS2_OK);
  struct { const char* name; void (*edit)(hs2_attn_desc*); hs2_status want; } cases[] = {
      {"batch 0", [](hs2_attn_desc* d) { d->batch = 0; }, HS2_EINVAL},
      {"batch -1", [](hs2_attn_desc* d) { d->batch = -1; }, HS2_EINVAL},
      {"batch INT_MAX", [](hs2_attn_desc* d) { d->batch = INT_MAX; }, HS2_EUNSUPPORTED},
      {"batch 2^24", [](hs2_attn_desc* d) { d->batch = 1 << 24; }, HS2_OK},
      {"batch 2^24+1", [](hs2_attn_desc* d) { d->batch = (1 << 24) + 1; }, HS2_EUNSUPPORTED},
      {"n_q 0", [](hs2_attn_desc* d) { d->n_q = 0; }, HS2_EINVAL},
      {"n_q 2 decode", [](hs2_attn_desc* d) { d->n_q = 2; }, HS2_EUNSUPPORTED},
      {"n_heads 0", [](hs2_attn_desc* d) { d->n_heads = 0; }, HS2_EINVAL},
      {"n_heads 33", [](hs2_attn_desc* d) { d->n_heads = 33; }, HS2_EUNSUPPORTED},
      {"n_heads 1", [](hs2_attn_desc* d) { d->n_heads = 1; }, HS2_OK},
      {"head_dim 0", [](hs2_attn_desc* d) { d->head_dim = 0; }, HS2_EINVAL},
      {"head_dim 64", [](hs2_attn_desc* d) { d->head_dim = 64; }, HS2_EUNSUPPORTED},
      {"tile_q 0", [](hs2_attn_desc* d) { d->tile_q = 0; }, HS2_EINVAL},
      {"tile_q -16", [](hs2_attn_desc* d) { d->tile_q = -16; }, HS2_EINVAL},
      {"k_top -1", [](hs2_attn_desc* d) { d->k_top = -1; }, HS2_EINVAL},
      {"k_top 0", [](hs2_attn_desc* d) { d->k_top = 0; }, HS2_OK},
      {"k_top 2048", [](hs2_attn_desc* d) { d->k_top = 2048; }, HS2_OK},
      {"k_top 2049", [](hs2_attn_desc* d) { d->k_top = 2049; }, HS2_EUNSUPPORTED},
      {"k_top INT_MIN", [](hs2_attn_desc* d) { d->k_top = INT_MIN; }, HS2_EINVAL},
      {"window -1", [](hs2_attn_desc* d) { d->window = -1; }, HS2_EINVAL},
      {"window 2049", [](hs2_attn_desc* d) { d->window = 2049; }, HS2_EUNSUPPORTED},
      {"causal 0", [](hs2_attn_desc* d) { d->causal = 0; }, HS2_EUNSUPPORTED},
      {"sm_scale 0", [](hs2_attn_desc* d) { d->sm_scale = 0.f; }, HS2_EINVAL},
      {"sm_scale -1", [](hs2_attn_desc* d) { d->sm_scale = -1.f; }, HS2_EINVAL},
      {"sm_scale nan", [](hs2_attn_desc* d) { d->sm_scale = NAN; }, HS2_EINVAL},
      {"sm_scale inf", [](hs2_attn_desc* d) { d->sm_scale = INFINITY; }, HS2_EINVAL},
      {"dtype 3", [](hs2_attn_desc* d) { set_dtype(d, 3); }, HS2_EINVAL},
      {"dtype -1", [](hs2_attn_desc* d) { set_dtype(d, -1); }, HS2_EINVAL},
      {"dtype INT_MAX", [](hs2_attn_desc* d) { set_dtype(d, INT_MAX); }, HS2_EINVAL},
      {"dtype f32", [](hs2_attn_desc* d) { set_dtype(d, HS2_F32); }, HS2_OK},
      {"fp8 ok", [](hs2_attn_desc* d) { set_dtype(d, HS2_FP8_E4M3); }, HS2_OK},
      {"fp8 k_scale 0", [](hs2_attn_desc* d) { set_dtype(d, HS2_FP8_E4M3); d->k_scale = 0.f; }, HS2_EINVAL},
      {"fp8 k_scale nan", [](hs2_attn_desc* d) { set_dtype(d, HS2_FP8_E4M3); d->k_scale = NAN; }, HS2_EINVAL},
      {"fp8 v_scale inf", [](hs2_attn_desc* d) { set_dtype(d, HS2_FP8_E4M3); d->v_scale = INFINITY; }, HS2_EINVAL},
      {"fp8 v_scale -2", [](hs2_attn_desc* d) { set_dtype(d, HS2_FP8_E4M3); d->v_scale = -2.f; }, HS2_EINVAL},
      {"bf16 ignores scales", [](hs2_attn_desc* d) { d->k_scale = NAN; d->v_scale = -1.f; }, HS2_OK},
      {"prefill bf16", [](hs2_attn_desc* d) { d->n_q = 128; d->tile_q = 64; }, HS2_OK},
      {"prefill tile 16", [](hs2_attn_desc* d) { d->n_q = 32; d->tile_q = 16; }, HS2_OK},
      {"prefill tile 8", [](hs2_attn_desc* d) { d->n_q = 8; d->tile_q = 8; }, HS2_EUNSUPPORTED},
      {"prefill n_q % tile", [](hs2_attn_desc* d) { d->n_q = 100; d->tile_q = 64; }, HS2_EINVAL},
      {"prefill f32", [](hs2_attn_desc* d) { d->n_q = 64; d->tile_q = 64; set_dtype(d, HS2_F32); }, HS2_EUNSUPPORTED},
      {"prefill fp8", [](hs2_attn_desc* d) { d->n_q = 64; d->tile_q = 64; set_dtype(d, HS2_FP8_E4M3); }, HS2_OK},
      {"prefill fp8 bad scale", [](hs2_attn_desc* d) { d->n_q = 64; d->tile_q = 64; set_dtype(d, HS2_FP8_E4M3); d->k_scale = 0.f; }, HS2_EINVAL},
      {"prefill rows 2^24", [](hs2_attn_desc* d) { d->batch = 1 << 11; d->n_q = 1 << 13; d->tile_q = 64; }, HS2_OK},
      {"prefill rows 2^25", [](hs2_attn_desc* d) { d->batch = 1 << 12; d->n_q = 1 << 13; d->tile_q = 64; }, HS2_EUNSUPPORTED},
      {"prefill n_q INT_MAX/64*64", [](hs2_attn_desc* d) { d->n_q = INT_MAX / 64 * 64; d->tile_q = 64; }, HS2_EUNSUPPORTED},
  };
  for (auto& c : cases) {
    hs2_attn_desc d = base;
    c.edit(&d);
    char name[96];
    snprintf(name, sizeof name, "desc %s", c.name);
    expect(name, check_desc(&d), c.want);
  }
}

void size_cases() {
  hs2_attn_desc d = decode_desc();
  expect("ws size > 0", workspace_bytes(&d, 262144) > 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("ws size cap 0", workspace_bytes(&d, 0) == 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("ws size cap max", workspace_bytes(&d, kMaxSelectCap) > 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("ws size cap max+1", workspace_bytes(&d, kMaxSelectCap + 1) == 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("ws size null", workspace_bytes(nullptr, 100) == 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  // The largest accepted problems: sizes well below 2^64 (no wrap-around).
  d.batch = 1 << 24;
  const size_t big = workspace_bytes(&d, kMaxSelectCap);
  expect("ws size 2^24 rows x max cap", big > ((size_t)1 << 40) && big < ((size_t)1 << 56) ? HS2_OK : HS2_EINVAL, HS2_OK);
  hs2_attn_desc p = prefill_desc();
  p.batch = 1 << 11; p.n_q = 1 << 13; p.tile_q = 16;
  const size_t bigp = workspace_bytes(&p, kMaxSelectCap);
  expect("ws size prefill 2^24 rows", bigp > ((size_t)1 << 40) && bigp < ((size_t)1 << 56) ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("layers ws 0 layers", layers_workspace_bytes(&d, 0) == 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("layers ws 65 layers", layers_workspace_bytes(&d, 65) == 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("layers ws 64 layers", layers_workspace_bytes(&d, 64) > 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("packed bytes 2048", bridge_packed_bytes(2048, 128) == 2048 * 256 * 2 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("packed bytes 100", bridge_packed_bytes(100, 128) == 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("packed bytes INT_MIN", bridge_packed_bytes(INT_MIN, 128) == 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
  expect("packed bytes head 64", bridge_packed_bytes(2048, 64) == 0 ? HS2_OK : HS2_EINVAL, HS2_OK);
}

// Arguments of a decode step; each case edits one of them.
struct Step {
  hs2_attn_desc d = decode_desc();
  const void *q = at<void>(A), *qs = nullptr, *k = at<void>(A), *v = at<void>(A);
  int64_t stride = 262144 * 128;
  const int32_t* ctx = at<int32_t>(A);
  int cap = 262144;
  const float *scores = at<float>(A), *lse_full = nullptr;
  const int32_t *top_idx = at<int32_t>(A), *top_cnt = at<int32_t>(A);
  const float *o = at<float>(A), *lse = nullptr;
  const void* ws = at<void>(A);
  size_t ws_bytes = 0;
  int block = 16;
  Step() { ws_bytes = workspace_bytes(&d, cap); }
  hs2_status step() const {
    return validate_step(&d, q, qs, k, v, stride, ctx, cap, scores, lse_full, top_idx, top_cnt, o,
                         lse, ws, ws_bytes);
  }
  hs2_status blocks() const {
    return validate_step_blocks(&d, block, q, qs, k, v, stride, ctx, cap, scores, lse_full,
                                top_idx, top_cnt, o, lse, ws, ws_bytes);
  }
  hs2_status noalloc(size_t scratch) const {
    return validate_step_noalloc(&d, q, qs, k, v, stride, ctx, cap, scores, lse_full, top_idx,
                                 top_cnt, o, lse, scratch);
  }
  hs2_status scores_call() const {
    return validate_full_attn_scores(&d, q, k, v, stride, ctx, cap, scores, o, lse, ws, ws_bytes);
  }
  hs2_status select() const {
    return validate_select_topk_window(&d, scores, ctx, cap, top_idx, top_cnt, ws, ws_bytes);
  }
  hs2_status select_blocks() const {
    return validate_select_topk_blocks(&d, block, scores, ctx, cap, top_idx, top_cnt, ws, ws_bytes);
  }
  hs2_status sparse() const {
    return validate_sparse_attn_gather(&d, q, k, v, stride, ctx, cap, top_idx, top_cnt, o, lse, ws,
                                       ws_bytes);
  }
};

void step_cases() {
  struct { const char* name; void (*edit)(Step*); hs2_status step, blocks, scores, select, sparse; } cases[] = {
      {"ok", [](Step*) {}, HS2_OK, HS2_OK, HS2_OK, HS2_OK, HS2_OK},
      {"desc null", [](Step* s) { s->d.batch = 0; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL},
      {"q null", [](Step* s) { s->q = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_OK, HS2_EINVAL},
      {"q misaligned", [](Step* s) { s->q = at<void>(M); }, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_OK, HS2_EALIGN},
      {"q_sparse misaligned", [](Step* s) { s->qs = at<void>(M); }, HS2_EALIGN, HS2_EALIGN, HS2_OK, HS2_OK, HS2_OK},
      {"k null", [](Step* s) { s->k = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_OK, HS2_EINVAL},
      {"v null", [](Step* s) { s->v = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_OK, HS2_EINVAL},
      {"v misaligned", [](Step* s) { s->v = at<void>(M); }, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_OK, HS2_EALIGN},
      {"ctx null", [](Step* s) { s->ctx = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL},
      {"ctx misaligned", [](Step* s) { s->ctx = at<int32_t>(M); }, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN},
      {"scores null", [](Step* s) { s->scores = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_OK},
      {"top_idx null", [](Step* s) { s->top_idx = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_OK, HS2_EINVAL, HS2_EINVAL},
      {"top_idx null k_top 0", [](Step* s) { s->top_idx = nullptr; s->d.k_top = 0; s->ws_bytes = workspace_bytes(&s->d, s->cap); },
       HS2_OK, HS2_OK, HS2_OK, HS2_OK, HS2_OK},
      {"top_cnt null", [](Step* s) { s->top_cnt = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_OK, HS2_EINVAL, HS2_EINVAL},
      {"o null", [](Step* s) { s->o = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_OK, HS2_OK, HS2_EINVAL},
      {"lse misaligned", [](Step* s) { s->lse = at<float>(M); }, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_OK, HS2_EALIGN},
      {"cap 0", [](Step* s) { s->cap = 0; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL},
      {"cap -5", [](Step* s) { s->cap = -5; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL},
      {"cap max+1", [](Step* s) { s->cap = kMaxSelectCap + 1; s->stride = (int64_t)s->cap * 128; },
       HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED},
      {"cap INT_MAX", [](Step* s) { s->cap = INT_MAX; s->stride = INT64_MAX / 2; },
       HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED},
      {"stride short", [](Step* s) { s->stride = 262144 * 128 - 8; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_OK, HS2_EINVAL},
      {"stride negative", [](Step* s) { s->stride = -128; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_OK, HS2_EINVAL},
      {"stride odd", [](Step* s) { s->stride = 262144 * 128 + 4; }, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_OK, HS2_EALIGN},
      {"fp8 stride 8", [](Step* s) { set_dtype(&s->d, HS2_FP8_E4M3); s->stride = 262144 * 128 + 8; s->ws_bytes = workspace_bytes(&s->d, s->cap); },
       HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_OK, HS2_EALIGN},
      {"ws short", [](Step* s) { s->ws_bytes -= 1; }, HS2_EWORKSPACE, HS2_EWORKSPACE, HS2_EWORKSPACE, HS2_EWORKSPACE, HS2_EWORKSPACE},
      {"ws null", [](Step* s) { s->ws = nullptr; }, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL, HS2_EINVAL},
      {"ws misaligned", [](Step* s) { s->ws = at<void>(M); }, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN, HS2_EALIGN},
      {"ws SIZE_MAX", [](Step* s) { s->ws_bytes = SIZE_MAX; }, HS2_OK, HS2_OK, HS2_OK, HS2_OK, HS2_OK},
      {"rows 2^24+1", [](Step* s) { s->d.batch = (1 << 24) + 1; s->ws_bytes = SIZE_MAX; },
       HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED, HS2_EUNSUPPORTED},
  };
  for (auto& c : cases) {
    Step s;
    c.edit(&s);
    char name[128];
    snprintf(name, sizeof name, "step %s", c.name);
    expect(name, s.step(), c.step);
    snprintf(name, sizeof name, "step_blocks %s", c.name);
    expect(name, s.blocks(), c.blocks);
    snprintf(name, sizeof name, "full_attn_scores %s", c.name);
    expect(name, s.scores_call(), c.scores);
    snprintf(name, sizeof name, "select_topk_window %s", c.name);
    expect(name, s.select(), c.select);
    snprintf(name, sizeof name, "select_topk_blocks %s", c.name);
    expect(name, s.select_blocks(), c.select);
    snprintf(name, sizeof name, "sparse_attn_gather %s", c.name);
    expect(name, s.sparse(), c.sparse);
  }
  // Block sizes (step and selector).
  struct { int block; int k_top; int cap; hs2_status want; } blocks[] = {
      {16, 1024, 262144, HS2_OK}, {1, 1024, 65536, HS2_OK}, {64, 1024, 262144, HS2_OK},
      {0, 1024, 262144, HS2_EINVAL}, {-16, 1024, 262144, HS2_EINVAL}, {24, 1024, 262144, HS2_EINVAL},
      {128, 1024, 262144, HS2_EINVAL}, {INT_MIN, 1024, 262144, HS2_EINVAL}, {64, 1000, 262144, HS2_EINVAL},
      {1, 1024, 65537, HS2_EUNSUPPORTED}, {2, 1024, 131072, HS2_OK}, {2, 1024, 131073, HS2_EUNSUPPORTED},
  };
  for (auto& b : blocks) {
    Step s;
    s.block = b.block; s.d.k_top = b.k_top; s.cap = b.cap; s.stride = (int64_t)b.cap * 128;
    s.ws_bytes = workspace_bytes(&s.d, s.cap);
    char name[96];
    snprintf(name, sizeof name, "block %d k_top %d cap %d", b.block, b.k_top, b.cap);
    expect(name, s.blocks(), b.want);
    expect(name, s.select_blocks(), b.want);
  }
  // The allocation-free step: arguments first, then the scratch size.
  Step s;
  expect("noalloc ok", s.noalloc((size_t)32 << 20), HS2_OK);
  expect("noalloc scratch short", s.noalloc(s.ws_bytes - 1), HS2_EWORKSPACE);
  s.q = at<void>(M);
  expect("noalloc misaligned before size", s.noalloc(0), HS2_EALIGN);
  Step t;
  t.d.causal = 2;
  expect("noalloc desc", t.noalloc((size_t)32 << 20), HS2_EUNSUPPORTED);
}

void layers_cases() {
  const hs2_attn_desc d = decode_desc();
  const size_t ws = layers_workspace_bytes(&d, 3);
  auto call = [&](const hs2_attn_desc& dd, int n, const void* ql, const void* w, size_t wb,
                  const float* lse) {
    return validate_sparse_attn_gather_layers(&dd, n, ql, at<void>(A), at<void>(A), 262144 * 128,
                                              at<int32_t>(A), 262144, at<int32_t>(A),
                                              at<int32_t>(A), at<float>(A), lse, w, wb);
  };
  expect("layers ok", call(d, 3, at<void>(A), at<void>(A), ws, nullptr), HS2_OK);
  expect("layers 0", call(d, 0, at<void>(A), at<void>(A), ws, nullptr), HS2_EINVAL);
  expect("layers 65", call(d, 65, at<void>(A), at<void>(A), SIZE_MAX, nullptr), HS2_EUNSUPPORTED);
  expect("layers q null", call(d, 3, nullptr, at<void>(A), ws, nullptr), HS2_EINVAL);
  expect("layers ws short", call(d, 3, at<void>(A), at<void>(A), ws - 1, nullptr), HS2_EWORKSPACE);
  expect("layers ws null", call(d, 3, at<void>(A), nullptr, ws, nullptr), HS2_EINVAL);
  expect("layers ws misaligned", call(d, 3, at<void>(A), at<void>(M), ws, nullptr), HS2_EALIGN);
  expect("layers lse misaligned", call(d, 3, at<void>(A), at<void>(A), ws, at<float>(M)), HS2_EALIGN);
  hs2_attn_desc f = d;
  set_dtype(&f, HS2_F32);
  expect("layers f32", call(f, 3, at<void>(A), at<void>(A), SIZE_MAX, nullptr), HS2_EUNSUPPORTED);
  const hs2_attn_desc p = prefill_desc();
  expect("layers prefill", call(p, 3, at<void>(A), at<void>(A), SIZE_MAX, nullptr), HS2_EUNSUPPORTED);
}

void swa_cases() {
  hs2_attn_desc d = prefill_desc();
  d.window = 128;
  auto call = [&](const hs2_attn_desc* dd, int odt, const void* o, int64_t stride, int cap) {
    return validate_swa_attention(dd, at<void>(A), at<void>(A), at<void>(A), stride,
                                  at<int32_t>(A), cap, o, odt, nullptr);
  };
  expect("swa ok bf16 out", call(&d, HS2_BF16, at<void>(A), 8192 * 128, 8192), HS2_OK);
  expect("swa ok f32 out", call(&d, HS2_F32, at<void>(A), 8192 * 128, 8192), HS2_OK);
  expect("swa null desc", call(nullptr, HS2_F32, at<void>(A), 8192 * 128, 8192), HS2_EINVAL);
  expect("swa o_dtype fp8", call(&d, HS2_FP8_E4M3, at<void>(A), 8192 * 128, 8192), HS2_EINVAL);
  expect("swa o_dtype 9", call(&d, 9, at<void>(A), 8192 * 128, 8192), HS2_EINVAL);
  expect("swa o_dtype -1", call(&d, -1, at<void>(A), 8192 * 128, 8192), HS2_EINVAL);
  expect("swa o null", call(&d, HS2_F32, nullptr, 8192 * 128, 8192), HS2_EINVAL);
  expect("swa o misaligned", call(&d, HS2_F32, at<void>(M), 8192 * 128, 8192), HS2_EALIGN);
  expect("swa stride short", call(&d, HS2_F32, at<void>(A), 8191 * 128, 8192), HS2_EINVAL);
  expect("swa stride odd", call(&d, HS2_F32, at<void>(A), 8192 * 128 + 4, 8192), HS2_EALIGN);
  expect("swa cap 0", call(&d, HS2_F32, at<void>(A), 8192 * 128, 0), HS2_EINVAL);
  hs2_attn_desc e = d;
  e.window = 0;
  expect("swa window 0", call(&e, HS2_F32, at<void>(A), 8192 * 128, 8192), HS2_EINVAL);
  e = d;
  set_dtype(&e, HS2_F32);
  expect("swa f32 cache", call(&e, HS2_F32, at<void>(A), 8192 * 128, 8192), HS2_EUNSUPPORTED);
  e = d;
  set_dtype(&e, 77);
  expect("swa dtype 77", call(&e, HS2_F32, at<void>(A), 8192 * 128, 8192), HS2_EINVAL);
  e = d;
  e.sm_scale = NAN;
  expect("swa sm_scale nan", call(&e, HS2_F32, at<void>(A), 8192 * 128, 8192), HS2_EINVAL);
}

void bridge_cases() {
  auto kv = [](const uint16_t* h, int64_t ldh, int64_t ld_kv, int M_, int dm, int hd) {
    return validate_bridge_kv(h, ldh, at<uint16_t>(A), at<uint16_t>(A), at<uint16_t>(A),
                              at<uint16_t>(A), ld_kv, M_, dm, hd);
  };
  expect("bridge ok", kv(at<uint16_t>(A), 2048, 128, 1 << 20, 2048, 128), HS2_OK);
  expect("bridge h null", kv(nullptr, 2048, 128, 1 << 20, 2048, 128), HS2_EINVAL);
  expect("bridge h misaligned", kv(at<uint16_t>(M), 2048, 128, 1 << 20, 2048, 128), HS2_EALIGN);
  expect("bridge M 0", kv(at<uint16_t>(A), 2048, 128, 0, 2048, 128), HS2_EINVAL);
  expect("bridge ldh short", kv(at<uint16_t>(A), 2047, 128, 16, 2048, 128), HS2_EINVAL);
  expect("bridge ldh odd", kv(at<uint16_t>(A), 2052, 128, 16, 2048, 128), HS2_EALIGN);
  expect("bridge ld_kv short", kv(at<uint16_t>(A), 2048, 64, 16, 2048, 128), HS2_EINVAL);
  expect("bridge d_model 100", kv(at<uint16_t>(A), 2048, 128, 16, 100, 128), HS2_EUNSUPPORTED);
  expect("bridge head 64", kv(at<uint16_t>(A), 2048, 128, 16, 2048, 64), HS2_EUNSUPPORTED);
  expect("bridge M INT_MAX", kv(at<uint16_t>(A), 2048, 128, INT_MAX, 2048, 128), HS2_OK);
  expect("bridge w_k null",
         validate_bridge_kv(at<uint16_t>(A), 2048, nullptr, at<uint16_t>(A), at<uint16_t>(A),
                            at<uint16_t>(A), 128, 16, 2048, 128), HS2_EINVAL);
  expect("bridge w_v misaligned",
         validate_bridge_kv(at<uint16_t>(A), 2048, at<uint16_t>(A), at<uint16_t>(M),
                            at<uint16_t>(A), at<uint16_t>(A), 128, 16, 2048, 128), HS2_EALIGN);
  expect("bridge packed ok",
         validate_bridge_kv_packed(at<uint16_t>(A), 2048, at<uint16_t>(A), at<uint16_t>(A),
                                   at<uint16_t>(A), 128, 16, 2048, 128), HS2_OK);
  expect("bridge packed null",
         validate_bridge_kv_packed(at<uint16_t>(A), 2048, nullptr, at<uint16_t>(A),
                                   at<uint16_t>(A), 128, 16, 2048, 128), HS2_EINVAL);
  expect("bridge packed misaligned",
         validate_bridge_kv_packed(at<uint16_t>(A), 2048, at<uint16_t>(M), at<uint16_t>(A),
                                   at<uint16_t>(A), 128, 16, 2048, 128), HS2_EALIGN);
  expect("pack ok", validate_bridge_pack_weights(at<uint16_t>(A), at<uint16_t>(A), 2048, 128,
                                                 at<uint16_t>(A)), HS2_OK);
  expect("pack null out", validate_bridge_pack_weights(at<uint16_t>(A), at<uint16_t>(A), 2048,
                                                       128, nullptr), HS2_EINVAL);
  expect("pack d_model 0", validate_bridge_pack_weights(at<uint16_t>(A), at<uint16_t>(A), 0, 128,
                                                        at<uint16_t>(A)), HS2_EINVAL);
  expect("pack d_model 96", validate_bridge_pack_weights(at<uint16_t>(A), at<uint16_t>(A), 96,
                                                         128, at<uint16_t>(A)), HS2_EUNSUPPORTED);
  auto dec = [](int rows, int64_t ldh, const int32_t* pos, int64_t stride, int cap) {
    return validate_bridge_kv_decode(at<uint16_t>(A), ldh, at<uint16_t>(A), rows, 2048, 128, pos,
                                     at<uint16_t>(A), at<uint16_t>(A), stride, cap);
  };
  expect("bridge decode ok", dec(4, 2048, at<int32_t>(A), 262144 * 128, 262144), HS2_OK);
  expect("bridge decode rows 0", dec(0, 2048, at<int32_t>(A), 262144 * 128, 262144), HS2_EINVAL);
  expect("bridge decode pos null", dec(4, 2048, nullptr, 262144 * 128, 262144), HS2_EINVAL);
  expect("bridge decode pos misaligned", dec(4, 2048, at<int32_t>(M), 262144 * 128, 262144), HS2_EALIGN);
  expect("bridge decode cap 0", dec(4, 2048, at<int32_t>(A), 262144 * 128, 0), HS2_EINVAL);
  expect("bridge decode stride short", dec(4, 2048, at<int32_t>(A), 262143 * 128, 262144), HS2_EINVAL);
  expect("bridge decode stride odd", dec(4, 2048, at<int32_t>(A), 262144 * 128 + 2, 262144), HS2_EALIGN);
  expect("bridge decode cap INT_MAX", dec(4, 2048, at<int32_t>(A), (int64_t)INT_MAX * 128, INT_MAX), HS2_OK);
}

}  // namespace

int main() {
  desc_cases();
  size_cases();
  step_cases();
  layers_cases();
  swa_cases();
  bridge_cases();
  printf("%d cases, %d mismatches\n", g_cases, g_bad);
  return g_bad == 0 ? 0 : 1;
}
