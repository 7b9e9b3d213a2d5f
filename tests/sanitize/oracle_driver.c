/*
 * Runs every entry point of the CPU oracle (oracle/moe_oracle.c) on a small
 * layer read from raw files, so that the oracle can be built and checked
 * under AddressSanitizer and UndefinedBehaviorSanitizer.  Test
 * infrastructure only.  Usage:
 *   oracle_driver DIR T d f E k wfmt
 * reads DIR/{x,wr,experts,shared,residual}.bin and writes DIR/out_<name>.bin.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

size_t orc_expert_bytes(int wfmt, int d, int f);
int orc_route(const float* x, int T, int d, const float* Wr, const float* bias, int E, int k, int32_t* ids,
              float* gates, double* logits);
int orc_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                int32_t* dest);
int orc_quant8(const float* x, int rows, int K, int8_t* q, float* s);
int orc_rmsnorm(const float* x, int T, int d, double eps, float* out);
int orc_dequant_expert(const uint8_t* blob, int wfmt, int d, int f, double* wg, double* wu, double* wd);
int orc_expert_ffn(const float* X, int M, int d, int f, const uint8_t* blob, int wfmt, int act_mode, double* Y,
                   double* G, double* U);
int orc_moe_layer(const float* x, int T, int d, int f, int E, int k, const float* Wr, const float* bias,
                  const uint8_t* const* experts, const uint8_t* shared, int wfmt, int act_mode, const float* residual,
                  const int32_t* tok, int n_tok, int32_t* ids, float* gates, int32_t* counts, int32_t* offsets,
                  int32_t* sorted_idx, int32_t* dest, float* out);

static void* slurp(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s.bin", dir, name);
    FILE* fp = fopen(path, "rb");
    if (!fp) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    void* p = malloc(bytes);
    if (!p || fread(p, 1, bytes, fp) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
    fclose(fp);
    return p;
}

static void spill(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/out_%s.bin", dir, name);
    FILE* fp = fopen(path, "wb");
    if (!fp || fwrite(p, 1, bytes, fp) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(fp);
}

#define CHECK(call) do { int rc_ = (call); if (rc_) { fprintf(stderr, "%s -> %d\n", #call, rc_); return 3; } } while (0)

int main(int argc, char** argv) {
    if (argc != 8) { fprintf(stderr, "usage: %s DIR T d f E k wfmt\n", argv[0]); return 2; }
    const char* dir = argv[1];
    const int T = atoi(argv[2]), d = atoi(argv[3]), f = atoi(argv[4]), E = atoi(argv[5]), k = atoi(argv[6]);
    const int wfmt = atoi(argv[7]);
    const size_t eb = orc_expert_bytes(wfmt, d, f);
    float* x = slurp(dir, "x", sizeof(float) * (size_t)T * d);
    float* wr = slurp(dir, "wr", sizeof(float) * (size_t)E * d);
    uint8_t* experts = slurp(dir, "experts", eb * (size_t)E);
    uint8_t* shared = slurp(dir, "shared", eb);
    float* res = slurp(dir, "residual", sizeof(float) * (size_t)T * d);
    const uint8_t** ptrs = malloc(sizeof(*ptrs) * (size_t)E);
    for (int e = 0; e < E; ++e) ptrs[e] = experts + (size_t)e * eb;

    int32_t* ids = malloc(sizeof(int32_t) * (size_t)T * k);
    float* gates = malloc(sizeof(float) * (size_t)T * k);
    double* logits = malloc(sizeof(double) * (size_t)T * E);
    CHECK(orc_route(x, T, d, wr, NULL, E, k, ids, gates, logits));
    spill(dir, "ids", ids, sizeof(int32_t) * (size_t)T * k);
    spill(dir, "gates", gates, sizeof(float) * (size_t)T * k);
    spill(dir, "logits", logits, sizeof(double) * (size_t)T * E);

    int32_t *counts = malloc(sizeof(int32_t) * E), *offsets = malloc(sizeof(int32_t) * (E + 1));
    int32_t *sorted = malloc(sizeof(int32_t) * (size_t)T * k), *dest = malloc(sizeof(int32_t) * (size_t)T * k);
    CHECK(orc_permute(ids, T, k, E, counts, offsets, sorted, dest));
    spill(dir, "sorted", sorted, sizeof(int32_t) * (size_t)T * k);

    int8_t* xq = malloc((size_t)T * d);
    float* sx = malloc(sizeof(float) * (size_t)T * (d / 32));
    CHECK(orc_quant8(x, T, d, xq, sx));
    spill(dir, "xq", xq, (size_t)T * d);

    float* xn = malloc(sizeof(float) * (size_t)T * d);
    CHECK(orc_rmsnorm(x, T, d, 1e-6, xn));
    spill(dir, "rmsnorm", xn, sizeof(float) * (size_t)T * d);

    double* w = malloc(sizeof(double) * 3 * (size_t)d * f);
    CHECK(orc_dequant_expert(ptrs[0], wfmt, d, f, w, w + (size_t)d * f, w + 2 * (size_t)d * f));
    spill(dir, "dequant", w, sizeof(double) * 3 * (size_t)d * f);

    double *Y = malloc(sizeof(double) * (size_t)T * d), *G = malloc(sizeof(double) * (size_t)T * f);
    double* U = malloc(sizeof(double) * (size_t)T * f);
    for (int mode = 0; mode < 2; ++mode) {
        CHECK(orc_expert_ffn(x, T, d, f, ptrs[1], wfmt, mode, Y, G, U));
        spill(dir, mode ? "ffn_q8" : "ffn_float", Y, sizeof(double) * (size_t)T * d);
    }
    float* out = malloc(sizeof(float) * (size_t)T * d);
    const int32_t tok[3] = {T - 1, 0, T / 2};
    for (int mode = 0; mode < 2; ++mode) {
        CHECK(orc_moe_layer(x, T, d, f, E, k, wr, NULL, ptrs, shared, wfmt, mode, res, NULL, T, ids, gates, counts,
                            offsets, sorted, dest, out));
        spill(dir, mode ? "layer_q8" : "layer_float", out, sizeof(float) * (size_t)T * d);
        CHECK(orc_moe_layer(x, T, d, f, E, k, wr, NULL, ptrs, NULL, wfmt, mode, NULL, tok, 3, ids, gates, counts,
                            offsets, sorted, dest, out));
        spill(dir, mode ? "subset_q8" : "subset_float", out, sizeof(float) * 3 * (size_t)d);
    }
    free(x); free(wr); free(experts); free(shared); free(res); free(ptrs); free(ids); free(gates); free(logits);
    free(counts); free(offsets); free(sorted); free(dest); free(xq); free(sx); free(xn); free(w); free(Y); free(G);
    free(U); free(out);
    return 0;
}
