// Drives every entry point of the C ABI (include/*.h) through valid and
// invalid arguments with fake device addresses (never dereferenced: the
// launches are stubs), so that an AddressSanitizer / UndefinedBehaviorSanitizer
// build of api.cpp runs each validation path. Exits 0 when every call returns
// the expected status; the sanitizers abort on any memory or UB error.
// Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "mamba_conv.h"
#include "mamba_scan.h"
#include "mamba_scan_bwd.h"
#include "mamba_ssd.h"

extern int g_stub_launches;
static int fails = 0;

// distinct, 256-byte aligned fake device addresses, 1 GiB apart
static void* P(int k) { return reinterpret_cast<void*>(uintptr_t(0x7F0000000000) + uintptr_t(k) * (1ull << 30)); }
static float* F(int k) { return static_cast<float*>(P(k)); }

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d (%s), expected %d: %s\n", what, got,
                 mamba_status_string(got), want, mamba_last_error());
    ++fails;
  }
}
static void expect_fail(int got, const char* what) {
  if (got == MAMBA_OK) {
    std::fprintf(stderr, "%s: accepted, expected a refusal\n", what);
    ++fails;
  } else if (std::strlen(mamba_last_error()) == 0) {
    std::fprintf(stderr, "%s: refused without a message\n", what);
    ++fails;
  }
}

static mamba_scan_desc SD(int64_t b, int64_t L, int64_t d, int64_t N, int io, uint32_t flags = 0,
                          int64_t G = 1) {
  mamba_scan_desc s;
  s.batch = b; s.seqlen = L; s.dim = d; s.dstate = N; s.io_dtype = io; s.flags = flags; s.ngroups = G;
  return s;
}

static int scan(const mamba_scan_desc* d, void* ws = nullptr, size_t wb = 0, int x = 1, int out = 9) {
  return mamba_scan_fwd(d, P(x), P(2), F(3), P(4), P(5), F(6), P(7), F(8), P(out), F(10), ws, wb, nullptr);
}

int main() {
  const int BF = MAMBA_BF16, FP = MAMBA_F32;
  // --- full-sequence scan
  mamba_scan_desc d = SD(2, 64, 512, 16, BF);
  expect(scan(&d), MAMBA_OK, "scan valid");
  expect(mamba_scan_fwd(&d, P(1), P(2), F(3), P(4), P(5), nullptr, nullptr, nullptr, P(9), nullptr,
                        nullptr, 0, nullptr), MAMBA_OK, "scan without optional inputs");
  expect_fail(scan(nullptr), "scan null desc");
  expect_fail(mamba_scan_fwd(&d, nullptr, P(2), F(3), P(4), P(5), F(6), P(7), F(8), P(9), F(10),
                             nullptr, 0, nullptr), "scan null x");
  expect_fail(scan(&d, nullptr, 0, 1, 1), "scan out == x");
  for (int64_t N : {3, 32, 0}) {
    mamba_scan_desc e = SD(2, 64, 512, N, BF);
    expect_fail(scan(&e), "scan bad dstate");
  }
  mamba_scan_desc neg = SD(-1, 64, 512, 16, BF);
  expect_fail(scan(&neg), "scan negative batch");
  mamba_scan_desc badio = SD(2, 64, 512, 16, 7);
  expect_fail(scan(&badio), "scan bad io dtype");
  mamba_scan_desc flag = SD(2, 64, 512, 16, BF, 1u << 24);
  expect_fail(scan(&flag), "scan unknown flag");
  mamba_scan_desc seg = SD(2, 64, 512, 16, BF, 4);  // four forced segments: needs a workspace
  const size_t need = mamba_scan_workspace_size(&seg);
  if (need == 0) { std::fprintf(stderr, "forced segments need a workspace\n"); ++fails; }
  expect_fail(scan(&seg), "scan missing workspace");
  expect_fail(scan(&seg, P(11), need - 1), "scan short workspace");
  expect_fail(scan(&seg, static_cast<char*>(P(11)) + 4, need), "scan misaligned workspace");
  expect_fail(scan(&seg, P(1), need), "scan workspace over x");
  expect(scan(&seg, P(11), need), MAMBA_OK, "scan with workspace");
  mamba_scan_desc grp = SD(2, 64, 512, 16, BF, 0, 3);
  expect_fail(scan(&grp), "scan groups not dividing dim");
  mamba_scan_desc grp2 = SD(2, 64, 512, 16, BF, 0, 2);
  expect(scan(&grp2), MAMBA_OK, "scan two groups");
  mamba_scan_desc zoh = SD(2, 64, 512, 16, FP, MAMBA_SCAN_ZOH);
  expect(scan(&zoh), MAMBA_OK, "scan zoh");
  mamba_scan_desc split = SD(2, 64, 512, 16, BF, MAMBA_SCAN_SPLIT_STATES);
  expect(scan(&split), MAMBA_OK, "scan split states");
  mamba_scan_desc split8 = SD(2, 64, 512, 8, BF, MAMBA_SCAN_SPLIT_STATES);
  expect_fail(scan(&split8), "split with dstate 8");
  mamba_scan_desc split_seg = SD(2, 64, 512, 16, BF, MAMBA_SCAN_SPLIT_STATES | 3);
  expect_fail(scan(&split_seg), "split with forced segments");
  mamba_scan_desc empty = SD(2, 0, 512, 16, BF);
  expect(scan(&empty), MAMBA_OK, "scan empty sequence");
  expect(mamba_scan_fwd(&d, reinterpret_cast<char*>(P(1)) + 1, P(2), F(3), P(4), P(5), F(6), P(7),
                        F(8), P(9), F(10), nullptr, 0, nullptr), MAMBA_ERR_INVALID_ARG, "scan odd x");
  // with h0
  expect(mamba_scan_fwd_init(&d, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), F(12), P(9), F(10),
                             nullptr, 0, nullptr), MAMBA_OK, "scan init");
  expect_fail(mamba_scan_fwd_init(&d, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), F(10), P(9),
                                  F(10), nullptr, 0, nullptr), "h0 == last_state");
  // strided
  mamba_scan_strides s{1024, 1024, 1024, 512, 64};
  expect(mamba_scan_fwd_strided(&d, &s, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), nullptr, P(9),
                                F(10), nullptr, 0, nullptr), MAMBA_OK, "scan strided");
  mamba_scan_strides bad{100, 1024, 1024, 512, 64};
  expect_fail(mamba_scan_fwd_strided(&d, &bad, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), nullptr,
                                     P(9), F(10), nullptr, 0, nullptr), "stride below the row");
  mamba_scan_strides huge{int64_t(1) << 27, 1024, 1024, 512, 64};
  expect_fail(mamba_scan_fwd_strided(&d, &huge, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), nullptr,
                                     P(9), F(10), nullptr, 0, nullptr), "stride too large");
  if (mamba_scan_workspace_size_strided(&seg, &s) == 0) { std::fprintf(stderr, "strided ws\n"); ++fails; }
  if (mamba_scan_workspace_size(nullptr) != 0) { std::fprintf(stderr, "ws of null desc\n"); ++fails; }
  // allocation-free scan
  expect(mamba_scan_fwd_noalloc(&seg, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), nullptr, P(9),
                                F(10), nullptr), MAMBA_OK, "noalloc with segments");
  mamba_scan_desc big = SD(4, 100000, 5120, 16, BF, 4000);
  expect(mamba_scan_fwd_noalloc(&big, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), nullptr, P(9),
                                F(10), nullptr), MAMBA_ERR_UNSUPPORTED, "noalloc plan too large");
  // --- one-token update
  mamba_scan_desc t = SD(8, 1, 512, 16, BF);
  expect(mamba_state_update(&t, F(1), P(2), P(3), F(4), P(5), P(6), F(7), P(8), F(9), P(10), nullptr),
         MAMBA_OK, "update valid");
  mamba_scan_desc t2 = SD(8, 2, 512, 16, BF);
  expect_fail(mamba_state_update(&t2, F(1), P(2), P(3), F(4), P(5), P(6), F(7), P(8), F(9), P(10),
                                 nullptr), "update seqlen 2");
  expect_fail(mamba_state_update(&t, F(1), P(2), P(3), F(4), P(5), P(6), F(7), P(8), F(9), P(2),
                                 nullptr), "update out == x");
  mamba_scan_strides ts{1024, 1024, 1024, 512, 32};
  expect(mamba_state_update_strided(&t, &ts, F(1), P(2), P(3), F(4), P(5), P(6), F(7), P(8), F(9),
                                    P(10), nullptr), MAMBA_OK, "update strided");
  // --- backward
  const size_t bw = mamba_scan_bwd_workspace_size(&d);
  expect(mamba_scan_bwd(&d, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), nullptr, P(11), F(12),
                        P(13), P(14), F(15), F(16), F(17), F(18), P(19), F(20), F(21), P(22), bw,
                        nullptr), MAMBA_OK, "bwd valid");
  expect_fail(mamba_scan_bwd(&d, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), nullptr, nullptr,
                             F(12), P(13), P(14), F(15), F(16), F(17), F(18), P(19), F(20), F(21),
                             P(22), bw, nullptr), "bwd without dout");
  expect_fail(mamba_scan_bwd(&d, P(1), P(2), F(3), P(4), P(5), F(6), P(7), F(8), nullptr, P(11),
                             F(12), P(13), P(14), F(15), F(16), F(17), F(18), P(19), F(20), F(21),
                             P(22), bw ? bw - 1 : 0, nullptr), "bwd short workspace");
  // --- convolution
  mamba_conv_desc c{2, 64, 512, 4, BF, 0};
  expect(mamba_conv1d_fwd(&c, P(1), F(2), F(3), P(4), P(5), P(6), nullptr), MAMBA_OK, "conv valid");
  mamba_conv_desc c0{2, 64, 512, 0, BF, 0};
  expect_fail(mamba_conv1d_fwd(&c0, P(1), F(2), F(3), P(4), P(5), P(6), nullptr), "conv width 0");
  expect_fail(mamba_conv1d_fwd(&c, P(1), F(2), F(3), P(4), P(1), P(6), nullptr), "conv out == xin");
  mamba_conv_desc cu{8, 1, 512, 4, BF, 0};
  expect(mamba_conv1d_update(&cu, P(1), P(2), F(3), F(4), P(5), nullptr), MAMBA_OK, "conv update");
  // --- Mamba-2 SSD
  mamba_ssd_desc sd{2, 300, 4, 64, 128, 2, BF, 0};
  const size_t sw = mamba_ssd_workspace_size(&sd);
  expect(mamba_ssd_fwd(&sd, P(1), P(2), F(3), P(4), P(5), F(6), F(7), nullptr, P(9), F(10), P(11), sw,
                       nullptr), MAMBA_OK, "ssd valid");
  mamba_ssd_desc sd32{2, 300, 4, 32, 128, 2, BF, 0};
  expect_fail(mamba_ssd_fwd(&sd32, P(1), P(2), F(3), P(4), P(5), F(6), F(7), nullptr, P(9), F(10),
                            P(11), sw, nullptr), "ssd headdim 32");
  mamba_ssd_desc sdg{2, 300, 4, 64, 128, 3, BF, 0};
  expect_fail(mamba_ssd_fwd(&sdg, P(1), P(2), F(3), P(4), P(5), F(6), F(7), nullptr, P(9), F(10),
                            P(11), sw, nullptr), "ssd groups not dividing heads");
  // --- status strings
  for (int k = -1; k < 6; ++k)
    if (!mamba_status_string(k) || !*mamba_status_string(k)) { std::fprintf(stderr, "status %d\n", k); ++fails; }
  if (g_stub_launches < 15) {
    std::fprintf(stderr, "only %d valid calls reached a launch\n", g_stub_launches);
    ++fails;
  }
  if (fails) { std::fprintf(stderr, "%d checks failed\n", fails); return 1; }
  std::printf("api driver: every case ran clean (%d launches reached)\n", g_stub_launches);
  return 0;
}
