/* Test driver for the CPU oracle (oracle/gpt2_oracle.c): reads a workload's
 * parameters and tokens from files, runs `steps` training steps (forward with
 * loss, backward, AdamW) and a few finite-difference gradients, and prints
 * each step's loss. The sanitizer test builds it together with the oracle
 * under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * usage: oracle_step_main V Vp maxT C L NH B T steps params.f32 tokens.i32
 * (tokens: steps x B x (T+1) int32; inputs [:, :T], targets [:, 1:]) */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    int V, Vp, maxT, C, L, NH, B, T;
} oracle_config;
typedef struct oracle_model oracle_model;
int64_t oracle_num_params(const oracle_config* c);
oracle_model* oracle_create(const oracle_config* cfg, const float* params);
void oracle_free(oracle_model* M);
int oracle_forward(oracle_model* M, const int* inputs, const int* targets, double* loss);
int oracle_backward(oracle_model* M);
void oracle_update(oracle_model* M, double lr, double b1, double b2, double eps, double wd,
                   int t);
int oracle_fd_grads(const oracle_config* cfg, const float* params, const int* inputs,
                    const int* targets, double h, int64_t start, int64_t count, double* fd);

static void* read_file(const char* path, size_t bytes) {
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(bytes);
    if (p && fread(p, 1, bytes, f) != bytes) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

int main(int argc, char** argv) {
    if (argc != 12) {
        fprintf(stderr, "usage: %s V Vp maxT C L NH B T steps params tokens\n", argv[0]);
        return 2;
    }
    oracle_config c = {atoi(argv[1]), atoi(argv[2]), atoi(argv[3]), atoi(argv[4]),
                       atoi(argv[5]), atoi(argv[6]), atoi(argv[7]), atoi(argv[8])};
    const int steps = atoi(argv[9]);
    const int64_t n = oracle_num_params(&c);
    const int64_t row = (int64_t)c.T + 1, per_step = (int64_t)c.B * row;
    float* params = (float*)read_file(argv[10], (size_t)n * sizeof(float));
    int* toks = (int*)read_file(argv[11], (size_t)(steps * per_step) * sizeof(int));
    int* in = (int*)malloc(sizeof(int) * c.B * c.T);
    int* tg = (int*)malloc(sizeof(int) * c.B * c.T);
    if (!params || !toks || !in || !tg) {
        fprintf(stderr, "cannot read inputs\n");
        return 2;
    }
    oracle_model* M = oracle_create(&c, params);
    if (!M) return 3;
    for (int s = 0; s < steps; s++) {
        for (int b = 0; b < c.B; b++)
            for (int t = 0; t < c.T; t++) {
                in[b * c.T + t] = toks[s * per_step + b * row + t];
                tg[b * c.T + t] = toks[s * per_step + b * row + t + 1];
            }
        double loss = 0;
        if (oracle_forward(M, in, tg, &loss) != 0 || oracle_backward(M) != 0) return 4;
        oracle_update(M, 1e-3, 0.9, 0.999, 1e-8, 0.1, s + 1);
        printf("loss %d %.17g\n", s + 1, loss);
    }
    /* finite differences over a few parameters (each thread steps a model copy) */
    double fd[8];
    if (oracle_fd_grads(&c, params, in, tg, 1e-4, 0, 8, fd) != 0) return 5;
    printf("fd %.17g\n", fd[0]);
    /* an out-of-range token is refused, not read */
    in[0] = c.V;
    double l2;
    if (oracle_forward(M, in, tg, &l2) != -1) return 6;
    oracle_free(M);
    free(params);
    free(toks);
    free(in);
    free(tg);
    return 0;
}
