// Host-side argument checking of every libspecv entry point, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the library (tests/test_host_sanitizers.py).
// Every call here is invalid or empty, so each must return its status without launching
// anything; device pointers are never dereferenced on the host, so stand-in addresses do.
// Exit status 0 when every call returned what was expected.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "specv.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, specv_last_error());
        ++failures;
    }
}

// either of two statuses (a check that may meet the missing device first)
void expect_any(const char* what, int got, int want1, int want2) {
    if (got != want1 && got != want2) expect(what, got, want1);
}

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

}  // namespace

int main() {
    const auto I = SPECV_ERR_INVALID_ARG, U = SPECV_ERR_UNSUPPORTED, W = SPECV_ERR_WORKSPACE;
    auto* i32 = static_cast<int32_t*>(fake(0x10000));
    auto* u32 = static_cast<uint32_t*>(fake(0x20000));
    void* dev = fake(0x30000);
    void* ws = fake(0x40000);
    const float nan = std::numeric_limits<float>::quiet_NaN();

    // status strings and the last-error text
    for (int s = -2; s < 8; ++s)
        if (specv_status_string(static_cast<specv_status>(s)) == nullptr) expect("status string", 1, 0);

    // mask
    expect("mask B<0", specv_build_tree_mask(i32, -1, 3, u32, i32, i32, nullptr), I);
    expect("mask K too large", specv_build_tree_mask(i32, 2, SPECV_MAX_NODES, u32, i32, i32, nullptr), I);
    expect("mask null parent", specv_build_tree_mask(nullptr, 2, 3, u32, i32, i32, nullptr), I);
    expect("mask empty", specv_build_tree_mask(i32, 0, 3, u32, i32, i32, nullptr), SPECV_OK);
    const int32_t IMAX = std::numeric_limits<int32_t>::max();
    expect("mask K INT_MAX", specv_build_tree_mask(i32, 2, IMAX, u32, i32, i32, nullptr), I);
    expect("mask B INT_MAX", specv_build_tree_mask(i32, IMAX, 3, u32, i32, i32, nullptr), I);

    // attention
    const size_t aw = specv_attn_workspace_bytes(2, 5, 8, 2, 128, 64);
    expect("attn Hq % Hkv", specv_tree_attn_verify(dev, dev, dev, i32, u32, 2, 5, 6, 4, 128, 64, 0.1f, SPECV_BF16,
                                                    dev, nullptr, ws, aw, nullptr), I);
    expect("attn D", specv_tree_attn_verify(dev, dev, dev, i32, u32, 2, 5, 8, 2, 96, 64, 0.1f, SPECV_BF16, dev,
                                            nullptr, ws, aw, nullptr), U);
    expect("attn Lmax < K + 1", specv_tree_attn_verify(dev, dev, dev, i32, u32, 2, 5, 8, 2, 128, 3, 0.1f, SPECV_BF16,
                                                        dev, nullptr, ws, aw, nullptr), I);
    expect("attn scale NaN", specv_tree_attn_verify(dev, dev, dev, i32, u32, 2, 5, 8, 2, 128, 64, nan, SPECV_BF16,
                                                     dev, nullptr, ws, aw, nullptr), I);
    // (the workspace plan reads the device's CU count, so without a device this is a HIP error)
    expect_any("attn workspace", specv_tree_attn_verify(dev, dev, dev, i32, u32, 2, 5, 8, 2, 128, 64, 0.1f,
                                                         SPECV_BF16, dev, nullptr, ws, aw > 0 ? aw - 1 : 0, nullptr),
               W, SPECV_ERR_HIP);
    expect("attn null q", specv_tree_attn_verify(nullptr, dev, dev, i32, u32, 2, 5, 8, 2, 128, 64, 0.1f, SPECV_BF16,
                                                  dev, nullptr, ws, aw, nullptr), I);
    expect("attn workspace query", static_cast<int>(specv_attn_workspace_bytes(-1, 5, 8, 2, 128, 64)), 0);
    expect("attn K INT_MAX", specv_tree_attn_verify(dev, dev, dev, i32, u32, 2, IMAX, 8, 2, 128, IMAX, 0.1f,
                                                     SPECV_BF16, dev, nullptr, ws, aw, nullptr), I);
    expect("attn B INT_MAX", specv_tree_attn_verify(dev, dev, dev, i32, u32, IMAX, 5, 8, 2, 128, 64, 0.1f,
                                                     SPECV_BF16, dev, nullptr, ws, aw, nullptr), I);
    expect("attn Hq INT_MAX", specv_tree_attn_verify(dev, dev, dev, i32, u32, 2, 5, IMAX, 1, 128, 64, 0.1f,
                                                      SPECV_BF16, dev, nullptr, ws, aw, nullptr), I);
    expect("attn workspace query K INT_MAX", static_cast<int>(specv_attn_workspace_bytes(2, IMAX, 8, 2, 128, 64)), 0);
    expect("attn workspace query B INT_MAX", static_cast<int>(specv_attn_workspace_bytes(IMAX, 5, 8, 2, 128, 64)), 0);
    expect("attn workspace query Hq INT_MAX",
           static_cast<int>(specv_attn_workspace_bytes(2, 5, IMAX, 1, 128, 64)), 0);

    // accept
    const size_t cw = specv_accept_workspace_bytes(4, 5, 1000, SPECV_BF16);
    auto accept = [&](int32_t B, int32_t K, int32_t V, float T, const void* draft, void* w, size_t wb,
                      int dtype = SPECV_BF16) {
        return specv_accept_resample(dev, draft, static_cast<specv_dtype>(dtype), i32, i32, B, K, V, T, 1, 0, i32,
                                     i32, i32, nullptr, nullptr, w, wb, nullptr);
    };
    expect("accept B<0", accept(-1, 5, 1000, 1.f, dev, ws, cw), I);
    expect("accept K", accept(4, SPECV_MAX_NODES, 1000, 1.f, dev, ws, cw), I);
    expect("accept V 0", accept(4, 5, 0, 1.f, dev, ws, cw), I);
    expect("accept V too large", accept(4, 5, SPECV_MAX_VOCAB + 1, 1.f, dev, ws, cw), I);
    expect("accept T<0", accept(4, 5, 1000, -1.f, dev, ws, cw), I);
    expect("accept T NaN", accept(4, 5, 1000, nan, dev, ws, cw), I);
    expect("accept T inf", accept(4, 5, 1000, INFINITY, dev, ws, cw), I);
    expect("accept dtype", accept(4, 5, 1000, 1.f, dev, ws, cw, 7), U);
    expect("accept no draft", accept(4, 5, 1000, 1.f, nullptr, ws, cw), I);
    expect("accept workspace", accept(4, 5, 1000, 1.f, dev, ws, cw > 0 ? cw - 1 : 0), W);
    expect("accept null workspace", accept(4, 5, 1000, 1.f, dev, nullptr, cw), W);
    expect("accept empty", accept(0, 5, 1000, 1.f, dev, ws, cw), SPECV_OK);
    expect("accept rule", specv_accept_resample_rule(dev, dev, SPECV_BF16, i32, i32, 4, 5, 1000, 1.f,
                                                     static_cast<specv_sibling_rule>(9), 1, 0, i32, i32, i32,
                                                     nullptr, nullptr, ws, cw, nullptr), I);
    expect("accept workspace query", static_cast<int>(specv_accept_workspace_bytes(4, 5, 0, SPECV_BF16)), 0);
    auto noalloc = [&](int B, int K, int V, float T, const void* d) {
        return specv_accept_resample_rule_noalloc(dev, d, SPECV_BF16, i32, i32, B, K, V, T,
                                                  SPECV_SIBLINGS_WITHOUT_REPLACEMENT, 1, 0, i32, i32, i32, nullptr,
                                                  nullptr, nullptr);
    };
    expect("noalloc B < 0", noalloc(-1, 5, 1000, 1.f, dev), I);
    expect("noalloc K INT_MAX", noalloc(4, IMAX, 1000, 1.f, dev), I);
    expect("noalloc T nan", noalloc(4, 5, 1000, std::nanf(""), dev), I);
    expect("noalloc draft null", noalloc(4, 5, 1000, 1.f, nullptr), I);
    expect("noalloc empty", noalloc(0, 5, 1000, 1.f, dev), SPECV_OK);
    expect("noalloc beyond its workspace", noalloc(256, 128, 262144, 1.f, dev), W);
    expect("accept K INT_MAX", accept(4, IMAX, 1000, 1.f, dev, ws, cw), I);
    expect("accept B INT_MAX", accept(IMAX, 5, 1000, 1.f, dev, ws, cw), I);
    expect("accept V INT_MAX", accept(4, 5, IMAX, 1.f, dev, ws, cw), I);
    expect("accept workspace query K INT_MAX",
           static_cast<int>(specv_accept_workspace_bytes(4, IMAX, 1000, SPECV_BF16)), 0);
    expect("accept workspace query B INT_MAX",
           static_cast<int>(specv_accept_workspace_bytes(IMAX, 5, 1000, SPECV_BF16)), 0);
    expect("accept workspace query V INT_MAX",
           static_cast<int>(specv_accept_workspace_bytes(4, 5, IMAX, SPECV_BF16)), 0);

    // KV commit
    expect("commit Lmax", specv_kv_commit(dev, dev, i32, i32, i32, 2, 5, 2, 128, 3, SPECV_BF16, i32, nullptr), I);
    expect("commit D", specv_kv_commit(dev, dev, i32, i32, i32, 2, 5, 2, 80, 64, SPECV_BF16, i32, nullptr), U);
    expect("commit null", specv_kv_commit(nullptr, dev, i32, i32, i32, 2, 5, 2, 128, 64, SPECV_BF16, i32, nullptr), I);
    expect("commit K INT_MAX", specv_kv_commit(dev, dev, i32, i32, i32, 2, IMAX, 2, 128, IMAX, SPECV_BF16, i32,
                                               nullptr), I);
    expect("commit B INT_MAX", specv_kv_commit(dev, dev, i32, i32, i32, IMAX, 5, 2, 128, 64, SPECV_BF16, i32,
                                               nullptr), I);
    expect("commit Hkv INT_MAX", specv_kv_commit(dev, dev, i32, i32, i32, 2, 5, IMAX, 128, 64, SPECV_BF16, i32,
                                                 nullptr), I);

    // tree expansion
    const size_t xw = specv_tree_expand_workspace_bytes(2, 4);
    auto expand = [&](int32_t F, int32_t V, int32_t k, float T, int32_t keep, int32_t nmax, size_t wb) {
        return specv_tree_expand(dev, SPECV_BF16, i32, 2, F, V, k, T, keep, nmax, i32, i32,
                                 static_cast<double*>(fake(0x50000)), i32, i32, ws, wb, nullptr);
    };
    expect("expand k 0", expand(4, 1000, 0, 1.f, 4, 32, xw), I);
    expect("expand k too large", expand(4, 1000, 17, 1.f, 4, 32, xw), I);
    expect("expand T 0", expand(4, 1000, 3, 0.f, 4, 32, xw), I);
    expect("expand nmax", expand(4, 1000, 3, 1.f, 4, SPECV_MAX_NODES + 1, xw), I);
    expect("expand workspace", expand(4, 1000, 3, 1.f, 4, 32, xw > 0 ? xw - 1 : 0), W);
    expect("expand F INT_MAX", expand(IMAX, 1000, 3, 1.f, 4, 32, xw), I);
    expect("expand V INT_MAX", expand(4, IMAX, 3, 1.f, 4, 32, xw), I);
    expect("expand k INT_MAX", expand(4, 1000, IMAX, 1.f, 4, 32, xw), I);
    expect("expand B INT_MAX", specv_tree_expand(dev, SPECV_BF16, i32, IMAX, 4, 1000, 3, 1.f, 4, 32, i32, i32,
                                                 static_cast<double*>(fake(0x50000)), i32, i32, ws, xw, nullptr), I);
    expect("expand workspace query", static_cast<int>(specv_tree_expand_workspace_bytes(IMAX, IMAX)), 0);

    // one target layer
    const size_t lw = specv_verify_layer_workspace_bytes(2, 5, 8, 2, 128, 64, 512);
    auto layer = [&](int32_t Hq, int32_t Hkv, int32_t D, int32_t Lmax, int32_t inter, float eps, float theta,
                     void* w, size_t wb) {
        return specv_verify_layer(dev, dev, dev, dev, dev, dev, dev, eps, theta, dev, dev, i32, u32, i32, 2, 5, Hq,
                                  Hkv, D, Lmax, inter, dev, w, wb, nullptr);
    };
    expect("layer inter % 64", layer(8, 2, 128, 64, 500, 1e-5f, 1e4f, ws, lw), I);
    expect("layer D", layer(8, 2, 96, 64, 512, 1e-5f, 1e4f, ws, lw), U);
    expect("layer eps", layer(8, 2, 128, 64, 512, 0.f, 1e4f, ws, lw), I);
    expect("layer theta", layer(8, 2, 128, 64, 512, 1e-5f, 1.f, ws, lw), I);
    expect("layer workspace", layer(8, 2, 128, 64, 512, 1e-5f, 1e4f, ws, lw > 0 ? lw - 1 : 0), W);
    expect("layer unaligned workspace", layer(8, 2, 128, 64, 512, 1e-5f, 1e4f, fake(0x40008), lw), W);
    expect("layer workspace query", static_cast<int>(specv_verify_layer_workspace_bytes(2, 5, 8, 2, 128, 64, 500)), 0);
    expect("layer inter INT_MAX", layer(8, 2, 128, 64, IMAX - 63, 1e-5f, 1e4f, ws, lw), I);
    expect("layer Hq INT_MAX", layer(IMAX, 1, 128, 64, 512, 1e-5f, 1e4f, ws, lw), I);
    expect("layer K INT_MAX", specv_verify_layer(dev, dev, dev, dev, dev, dev, dev, 1e-5f, 1e4f, dev, dev, i32, u32,
                                                 i32, 2, IMAX, 8, 2, 128, IMAX, 512, dev, ws, lw, nullptr), I);
    expect("layer B INT_MAX", specv_verify_layer(dev, dev, dev, dev, dev, dev, dev, 1e-5f, 1e4f, dev, dev, i32, u32,
                                                 i32, IMAX, 5, 8, 2, 128, 64, 512, dev, ws, lw, nullptr), I);
    expect("layer workspace query inter INT_MAX",
           static_cast<int>(specv_verify_layer_workspace_bytes(2, 5, 8, 2, 128, 64, IMAX - 63)), 0);
    expect("layer workspace query K INT_MAX",
           static_cast<int>(specv_verify_layer_workspace_bytes(2, IMAX, 8, 2, 128, IMAX, 512)), 0);
    expect("layer workspace query B INT_MAX",
           static_cast<int>(specv_verify_layer_workspace_bytes(IMAX, 5, 8, 2, 128, 64, 512)), 0);

    // the same layer on packed weights, and packing
    expect("packed layer K INT_MAX", specv_verify_layer_packed(dev, dev, dev, dev, dev, dev, dev, 1e-5f, 1e4f, dev,
                                                               dev, i32, u32, i32, 2, IMAX, 8, 2, 128, IMAX, 512,
                                                               dev, ws, lw, nullptr), I);
    expect("packed layer inter % 64", specv_verify_layer_packed(dev, dev, dev, dev, dev, dev, dev, 1e-5f, 1e4f, dev,
                                                                dev, i32, u32, i32, 2, 5, 8, 2, 128, 64, 500, dev, ws,
                                                                lw, nullptr), I);
    expect("pack N INT_MAX", specv_pack_weights(dev, IMAX, 64, fake(0x90000), nullptr), I);
    expect("pack K INT_MAX", specv_pack_weights(dev, 64, IMAX, fake(0x90000), nullptr), I);
    expect("pack N negative", specv_pack_weights(dev, -32, 64, fake(0x90000), nullptr), I);
    expect("pack NULL", specv_pack_weights(nullptr, 64, 64, fake(0x90000), nullptr), I);

    // read probe (measurement aid)
    const size_t sw = static_cast<size_t>(specv_read_probe_sink_words());
    expect("probe empty", specv_read_probe(nullptr, 0, nullptr, 0, nullptr), SPECV_OK);
    expect("probe NULL buf", specv_read_probe(nullptr, 1024, u32, sw, nullptr), I);
    expect("probe misaligned", specv_read_probe(fake(0x30008), 1024, u32, sw, nullptr), I);
    expect("probe size", specv_read_probe(dev, 1000, u32, sw, nullptr), I);
    expect("probe sink", specv_read_probe(dev, 1024, u32, sw - 1, nullptr), I);
    expect("probe huge size", specv_read_probe(dev, SIZE_MAX & ~size_t(15), u32, 0, nullptr), I);
    // the bounds record of the product build
    expect("bounds record", static_cast<int>(specv_debug_bounds(0)), -1);

    std::printf("%s: %d failing checks\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
