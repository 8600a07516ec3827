// Every argument check of the C ABI (block_scaled_fp4_pre_amd/csrc/validate.cpp),
// built for the host on its own and run under the address and
// undefined-behaviour sanitizers by tests/test_abi_sanitized.py.  abi.cpp runs
// exactly these checks before any HIP call, so each error path of the ABI is
// exercised here without a GPU.  Prints one line per failed expectation and
// "ok <cases>" at the end; the exit status is the number of failures (capped).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "validate.h"

namespace {

int g_cases = 0, g_fail = 0;

void expect(int got, int want, const char* what, int line) {
  ++g_cases;
  if (got != want) {
    ++g_fail;
    printf("FAIL line %d: %s: got %d want %d\n", line, what, got, want);
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

moe_w4a4_cfg base_cfg() {
  moe_w4a4_cfg c;
  memset(&c, 0, sizeof(c));
  c.hidden = 256;
  c.inter = 128;
  c.num_experts = 8;
  c.topk = 2;
  c.max_tokens = 16;
  c.group_size = 32;
  c.mma_type = MOE_MMA_MXF4_X_MXF4;
  c.activation = MOE_ACT_SWIGLU;
  return c;
}

// Distinct, suitably aligned addresses that are never dereferenced.
const void* P(uintptr_t a) { return reinterpret_cast<const void*>(a); }
const uintptr_t A = uintptr_t(1) << 20;

void cfg_checks() {
  moe_w4a4_cfg c = base_cfg();
  EXPECT(moe::check_cfg(&c), MOE_OK);
  EXPECT(moe::check_cfg(nullptr), MOE_EINVAL);
  struct Case { int32_t moe_w4a4_cfg::*field; int32_t value; int want; };
  const Case cases[] = {
      {&moe_w4a4_cfg::hidden, 0, MOE_EINVAL},        {&moe_w4a4_cfg::hidden, -256, MOE_EINVAL},
      {&moe_w4a4_cfg::hidden, 128, MOE_EUNSUPPORTED}, {&moe_w4a4_cfg::hidden, 4000, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::hidden, 1 << 17, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::inter, 0, MOE_EINVAL},         {&moe_w4a4_cfg::inter, 100, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::inter, 1 << 17, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::num_experts, 0, MOE_EINVAL},   {&moe_w4a4_cfg::num_experts, 513, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::num_experts, 512, MOE_OK},     {&moe_w4a4_cfg::num_experts, 1, MOE_OK},
      {&moe_w4a4_cfg::topk, 0, MOE_EINVAL},          {&moe_w4a4_cfg::topk, 17, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::topk, 16, MOE_OK},
      {&moe_w4a4_cfg::max_tokens, -1, MOE_EINVAL},   {&moe_w4a4_cfg::max_tokens, 0, MOE_OK},
      {&moe_w4a4_cfg::max_tokens, 1 << 30, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::group_size, 16, MOE_EUNSUPPORTED}, {&moe_w4a4_cfg::group_size, 0, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::mma_type, 2, MOE_EUNSUPPORTED}, {&moe_w4a4_cfg::mma_type, -1, MOE_EUNSUPPORTED},
      {&moe_w4a4_cfg::mma_type, MOE_MMA_FP8_X_MXF4, MOE_OK},
      {&moe_w4a4_cfg::activation, 1, MOE_EUNSUPPORTED},
  };
  for (const Case& k : cases) {
    moe_w4a4_cfg d = base_cfg();
    d.*(k.field) = k.value;
    expect(moe::check_cfg(&d), k.want, "check_cfg field", k.value);
  }
  // max_tokens * topk must stay below 2^31
  moe_w4a4_cfg big = base_cfg();
  big.topk = 16;
  big.max_tokens = (1 << 27) - 1;
  EXPECT(moe::check_cfg(&big), MOE_OK);
  big.max_tokens = 1 << 27;
  EXPECT(moe::check_cfg(&big), MOE_EUNSUPPORTED);
}

void layout_checks() {
  // Regions are 256-byte aligned, in order, disjoint, and inside the total;
  // the prepared buffer ends with the read-ahead tail.
  const int shapes[][5] = {{256, 128, 8, 2, 16}, {4096, 2048, 256, 6, 512}, {768, 384, 5, 3, 0},
                           {4096, 2048, 256, 6, 16384}, {512, 512, 512, 16, 2000}};
  for (const auto& s : shapes) {
    for (int mma = 0; mma < 2; ++mma) {
      moe_w4a4_cfg c = base_cfg();
      c.hidden = s[0];
      c.inter = s[1];
      c.num_experts = s[2];
      c.topk = s[3];
      c.max_tokens = s[4];
      c.mma_type = mma;
      EXPECT(moe::check_cfg(&c), MOE_OK);
      const moe::PreparedLayout p = moe::prepared_layout(&c);
      const uint64_t H = c.hidden, I = c.inter, E = c.num_experts;
      const uint64_t pr[4][2] = {{p.w1c, E * 2 * I * H / 2}, {p.w1s, E * 2 * I * H / 32},
                                 {p.w2c, E * H * I / 2}, {p.w2s, E * H * I / 32}};
      uint64_t end = 0;
      for (const auto& r : pr) {
        expect(r[0] % 256 == 0 && r[0] >= end, 1, "prepared region aligned and after the previous", s[0]);
        end = r[0] + r[1];
      }
      expect(p.total >= end + moe::kPreparedTailBytes, 1, "prepared tail", s[0]);
      const moe_w4a4_ws_layout L = moe::ws_layout(&c);
      const uint64_t R = (uint64_t)c.max_tokens * c.topk, ab = mma ? 2 : 1;
      const uint64_t wr[][2] = {{L.mega, moe::kMegaStateBytes}, {L.xq, c.max_tokens * H / 2 * ab},
                                {L.xsf, c.max_tokens * H / 32},
                                {L.counts, E * 4}, {L.offsets, (E + 1) * 4}, {L.sorted_rows, R * 4},
                                {L.pos, R * 4}, {L.hist, (R + 1023) / 1024 * E * 4}, {L.hq, R * I / 2 * ab},
                                {L.hsf, R * I / 32}, {L.y, R * H * 2}, {L.tiles, (R / 16 + E + 1) * 8},
                                {L.num_tiles, 4}, {L.xsf_planes, R * H / 32}};
      end = 0;
      for (const auto& r : wr) {
        expect(r[0] % 256 == 0 && r[0] >= end, 1, "workspace region aligned and after the previous", s[0]);
        end = r[0] + r[1];
      }
      expect(L.total >= end && L.total % 256 == 0, 1, "workspace total", s[0]);
      expect(L.mega == 0, 1, "the single-launch state region comes first", s[0]);
    }
  }
}

void quantize_checks() {
  bool noop = true;
  EXPECT(moe::check_quantize_args(0, P(A), 4, 64, P(A), P(A), &noop), MOE_OK);
  expect(noop, 0, "quantize noop flag", 0);
  EXPECT(moe::check_quantize_args(1, P(A), 4, 64, P(A), P(A), &noop), MOE_OK);
  EXPECT(moe::check_quantize_args(2, P(A), 4, 64, P(A), P(A), &noop), MOE_EUNSUPPORTED);
  EXPECT(moe::check_quantize_args(-1, P(A), 4, 64, P(A), P(A), &noop), MOE_EUNSUPPORTED);
  EXPECT(moe::check_quantize_args(0, P(A), -1, 64, P(A), P(A), &noop), MOE_EINVAL);
  EXPECT(moe::check_quantize_args(0, P(A), 4, 0, P(A), P(A), &noop), MOE_EINVAL);
  EXPECT(moe::check_quantize_args(0, P(A), 4, -32, P(A), P(A), &noop), MOE_EINVAL);
  EXPECT(moe::check_quantize_args(0, P(A), 4, 48, P(A), P(A), &noop), MOE_EUNSUPPORTED);
  EXPECT(moe::check_quantize_args(0, nullptr, 0, 64, nullptr, nullptr, &noop), MOE_OK);
  expect(noop, 1, "quantize of zero rows is a no-op", 0);
  EXPECT(moe::check_quantize_args(0, nullptr, 4, 64, P(A), P(A), &noop), MOE_EINVAL);
  EXPECT(moe::check_quantize_args(0, P(A), 4, 64, nullptr, P(A), &noop), MOE_EINVAL);
  EXPECT(moe::check_quantize_args(0, P(A), 4, 64, P(A), nullptr, &noop), MOE_EINVAL);
  EXPECT(moe::check_quantize_args(0, P(A + 8), 4, 64, P(A), P(A), &noop), MOE_EINVAL);
  EXPECT(moe::check_quantize_args(0, P(A), 4, 64, P(A + 4), P(A), &noop), MOE_EINVAL);
  EXPECT(moe::check_quantize_args(0, P(A), 4, 64, P(A), P(A + 1), &noop), MOE_OK);   // scale bytes: any address
  EXPECT(moe::check_quantize_args(0, P(A), (int64_t)1 << 40, 64, P(A), P(A), &noop), MOE_EUNSUPPORTED);
}

void prepare_checks() {
  moe_w4a4_cfg c = base_cfg();
  const size_t need = moe::prepared_layout(&c).total;
  EXPECT(moe::check_prepare_args(&c, P(A), P(A), P(A), P(A), P(A), need), MOE_OK);
  EXPECT(moe::check_prepare_args(&c, P(A), P(A), P(A), P(A), P(A), need - 1), MOE_EWORKSPACE);
  EXPECT(moe::check_prepare_args(&c, P(A), P(A), P(A), P(A), P(A), 0), MOE_EWORKSPACE);
  EXPECT(moe::check_prepare_args(nullptr, P(A), P(A), P(A), P(A), P(A), need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, nullptr, P(A), P(A), P(A), P(A), need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, P(A), nullptr, P(A), P(A), P(A), need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, P(A), P(A), nullptr, P(A), P(A), need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, P(A), P(A), P(A), nullptr, P(A), need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, P(A), P(A), P(A), P(A), nullptr, need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, P(A + 8), P(A), P(A), P(A), P(A), need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, P(A), P(A), P(A + 8), P(A), P(A), need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, P(A), P(A), P(A), P(A), P(A + 64), need), MOE_EINVAL);
  EXPECT(moe::check_prepare_args(&c, P(A), P(A + 1), P(A), P(A + 3), P(A), need), MOE_OK);
  moe_w4a4_cfg bad = base_cfg();
  bad.mma_type = 7;
  EXPECT(moe::check_prepare_args(&bad, P(A), P(A), P(A), P(A), P(A), need), MOE_EUNSUPPORTED);
}

void stage_checks() {
  moe_w4a4_cfg c = base_cfg();
  const size_t ws = moe::ws_layout(&c).total;
  const uint32_t ALL = MOE_STAGE_ALL;
  bool noop = true;
  auto run = [&](const void* prep, int32_t T, const void* x, const void* ids, const void* w, const void* out,
                 const void* wsp, size_t wsb, uint32_t stages, const void* acc) {
    return moe::check_stage_args(&c, prep, T, x, ids, w, out, wsp, wsb, stages, acc, &noop);
  };
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_OK);
  expect(noop, 0, "forward noop flag", 0);
  EXPECT(run(P(A), 16, P(A), P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_OK);      // at capacity
  EXPECT(run(P(A), 17, P(A), P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_ECAPACITY);
  EXPECT(run(P(A), -1, P(A), P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A), P(A), ws - 1, ALL, nullptr), MOE_EWORKSPACE);
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A), nullptr, ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A), P(A + 128), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A), P(A), ws, 64, nullptr), MOE_EINVAL);     // unknown stage bit
  // nothing to do: no pointer is looked at
  EXPECT(run(nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0, ALL, nullptr), MOE_OK);
  expect(noop, 1, "zero tokens is a no-op", 0);
  EXPECT(run(nullptr, 4, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr), MOE_OK);
  expect(noop, 1, "no stages is a no-op", 0);
  // each stage needs only its own pointers
  EXPECT(run(P(A), 4, nullptr, P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, P(A + 2), P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(nullptr, 4, P(A), nullptr, nullptr, nullptr, P(A), ws, MOE_STAGE_QUANT, nullptr), MOE_OK);
  EXPECT(run(P(A), 4, P(A), nullptr, P(A), P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, P(A), P(A + 2), P(A), P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(nullptr, 4, nullptr, P(A), nullptr, nullptr, P(A), ws, MOE_STAGE_ROUTE, nullptr), MOE_OK);
  EXPECT(run(nullptr, 4, P(A), P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A + 16), 4, P(A), P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(nullptr, 4, nullptr, nullptr, nullptr, nullptr, P(A), ws, MOE_STAGE_GEMM2, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, nullptr, nullptr, nullptr, nullptr, P(A), ws, MOE_STAGE_GEMM1, nullptr), MOE_OK);
  EXPECT(run(P(A), 4, P(A), P(A), nullptr, P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, P(A), P(A), P(A + 2), P(A), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, P(A), P(A), P(A), nullptr, P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A + 8), P(A), ws, ALL, nullptr), MOE_EINVAL);
  EXPECT(run(nullptr, 4, nullptr, nullptr, P(A), P(A), P(A), ws, MOE_STAGE_COMBINE, nullptr), MOE_OK);
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A), P(A), ws, ALL, P(A)), MOE_OK);
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A), P(A), ws, ALL, P(A + 4)), MOE_EINVAL);
  // a bad configuration is reported before anything else
  c.group_size = 64;
  EXPECT(run(P(A), 4, P(A), P(A), P(A), P(A), P(A), ws, ALL, nullptr), MOE_EUNSUPPORTED);
  EXPECT(moe::check_stage_args(nullptr, P(A), 4, P(A), P(A), P(A), P(A), P(A), ws, ALL, nullptr, &noop),
         MOE_EINVAL);
}

void mega_checks() {
  // The single-launch forward: MXFP4 or fp8xfp4, H and I of 512, 1024, 2048
  // or 4096, at most MOE_MEGA_MAX_ROWS routed rows.  NVFP4: refused.
  moe_w4a4_cfg c = base_cfg();
  c.hidden = 4096;
  c.inter = 2048;
  c.num_experts = 256;
  c.topk = 6;
  c.max_tokens = 64;
  EXPECT(moe::check_mega_args(&c, 42), MOE_OK);               // 252 rows
  EXPECT(moe::check_mega_args(&c, 43), MOE_EUNSUPPORTED);     // 258 rows
  EXPECT(moe::check_mega_args(&c, 0), MOE_OK);
  c.topk = 1;
  EXPECT(moe::check_mega_args(&c, 256), MOE_OK);
  EXPECT(moe::check_mega_args(&c, 257), MOE_EUNSUPPORTED);
  c.topk = 6;
  c.mma_type = MOE_MMA_FP8_X_MXF4;
  EXPECT(moe::check_mega_args(&c, 42), MOE_OK);
  EXPECT(moe::check_mega_args(&c, 43), MOE_EUNSUPPORTED);
  c.mma_type = MOE_MMA_NVF4_X_NVF4;
  EXPECT(moe::check_mega_args(&c, 1), MOE_EUNSUPPORTED);
  c.mma_type = MOE_MMA_MXF4_X_MXF4;
  const int shapes[][2] = {{4096, 2048}, {512, 512}, {2048, 1024}, {4096, 4096}};
  for (const auto& s : shapes) {
    c.hidden = s[0];
    c.inter = s[1];
    expect(moe::check_mega_args(&c, 1), MOE_OK, "supported shape", s[0] + s[1]);
  }
  const int bad[][2] = {{768, 512}, {512, 384}, {8192, 512}, {512, 8192}, {256, 512},
                        {1536, 512}, {512, 1536}, {3072, 2048}, {4096, 2560}, {3584, 512}};
  for (const auto& s : bad) {
    c.hidden = s[0];
    c.inter = s[1];
    expect(moe::check_mega_args(&c, 1), MOE_EUNSUPPORTED, "unsupported shape", s[0] + s[1]);
  }
}

}  // namespace

int main() {
  cfg_checks();
  layout_checks();
  quantize_checks();
  prepare_checks();
  stage_checks();
  mega_checks();
  // A heap copy of a layout, read back: gives the address sanitizer real
  // allocations to watch next to the stack-only checks above.
  std::vector<moe_w4a4_ws_layout> v(3);
  moe_w4a4_cfg c = base_cfg();
  for (auto& l : v) l = moe::ws_layout(&c);
  expect(v[2].total == v[0].total, 1, "layout copies agree", 0);
  printf("ok %d cases, %d failed\n", g_cases, g_fail);
  return g_fail > 100 ? 100 : g_fail;
}
