/*
 * A plain C consumer of libdita: the library's C ABI used without Python.
 *
 *   dita_c_client check       host-only: version, status strings, cache sizing,
 *                             argument validation and the planner (no GPU call)
 *   dita_c_client run <dir>   reads a problem from <dir> (written by the test),
 *                             runs its rank-steps on the GPU through
 *                             dita_attn_step, writes each step's O and LSE back
 *
 * Problem files (little-endian): meta.txt "B H D Nq P steps dtype"; nk.txt P key
 * counts; q.bin; k<p>.bin, v<p>.bin; mask<s>.bin (P bytes per step).  Outputs:
 * o<s>.bin, lse<s>.bin and info<s>.txt "n_fresh n_reused".
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/dita.h"

#define FAKE_DEV ((void*)(uintptr_t)0x7F0000000000ull)

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int fail(const char* what, int st) {
  fprintf(stderr, "%s: %s (%d)\n", what, dita_status_str(st), st);
  return 1;
}

static int expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d want %d\n", what, got, want);
    return 1;
  }
  return 0;
}

static int check(void) {
  int bad = 0;
  printf("version %d\n", dita_version());
  bad |= expect("version", dita_version() >= 100, 1);
  bad |= expect("status ok", strcmp(dita_status_str(DITA_OK), "ok"), 0);
  dita_shape sh = {1, 2, 128, DITA_BF16, 100, 0.0f};
  /* a slot is O then LSE, each rounded up to 256 bytes */
  const size_t slot = align256((size_t)2 * 100 * 128 * 2) + align256((size_t)2 * 100 * 4);
  const size_t n = dita_state_cache_bytes(&sh, 3);
  printf("cache_bytes %zu\n", n);
  bad |= expect("cache bytes", n == 3 * slot, 1);
  dita_state_cache* c = NULL;
  bad |= expect("init", dita_state_cache_init(&c, &sh, 3, FAKE_DEV, n), DITA_OK);
  bad |= expect("init small", dita_state_cache_init(&c, &sh, 3, FAKE_DEV, n - 1), DITA_ERR_SIZE);
  int valid = 7;
  int64_t stamp = 7;
  bad |= expect("info", dita_state_cache_info(c, 1, &valid, &stamp), DITA_OK);
  bad |= expect("empty slot", valid == 0 && stamp == -1, 1);
  /* reuse of an empty slot is refused before any launch */
  const void* ks[3] = {(char*)FAKE_DEV + (64 << 20), (char*)FAKE_DEV + (65 << 20), (char*)FAKE_DEV + (66 << 20)};
  const int64_t nk[3] = {64, 64, 64};
  const uint8_t mask[3] = {0, 1, 0};
  bad |= expect("reuse empty", dita_attn_step(c, (char*)FAKE_DEV + (60 << 20), ks, ks, nk, mask, 0,
                                              (char*)FAKE_DEV + (61 << 20), (float*)((char*)FAKE_DEV + (62 << 20)),
                                              NULL, NULL), DITA_ERR_STATE);
  /* the planner: radius 1 around partition 0 of 5, anchors every 4th step */
  dita_plan plan = {5, 0, DITA_PLAN_DIST, 1, 0, 0, 4, 1, 0};
  uint8_t out[5];
  bad |= expect("plan", dita_plan_mask(&plan, NULL, 3, out), DITA_OK);
  printf("plan %d%d%d%d%d\n", out[0], out[1], out[2], out[3], out[4]);
  bad |= expect("plan mask", memcmp(out, "\0\0\1\1\1", 5), 0);
  bad |= expect("anchor", dita_plan_mask(&plan, NULL, 4, out) == DITA_OK && !(out[2] | out[3] | out[4]), 1);
  uint64_t bits = 0;
  bad |= expect("plan bits", dita_plan_bits(&plan, NULL, 3, &bits), DITA_OK);
  bad |= expect("bits value", bits == 0x1Cu, 1);
  dita_state_cache_free(c);
  printf(bad ? "check FAILED\n" : "check ok\n");
  return bad;
}

static void* read_file(const char* dir, const char* name, size_t* size) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  fseek(f, 0, SEEK_END);
  const long len = ftell(f);
  fseek(f, 0, SEEK_SET);
  void* buf = malloc(len > 0 ? (size_t)len : 1);
  if (buf && fread(buf, 1, (size_t)len, f) != (size_t)len) {
    free(buf);
    buf = NULL;
  }
  fclose(f);
  if (size) *size = (size_t)len;
  return buf;
}

static int write_file(const char* dir, const char* name, const void* data, size_t size) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const int ok = fwrite(data, 1, size, f) == size;
  fclose(f);
  return !ok;
}

static void* to_device(const void* host, size_t size) {
  void* d = NULL;
  if (hipMalloc(&d, size) != hipSuccess) return NULL;
  if (hipMemcpy(d, host, size, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

static int run(const char* dir) {
  int B, H, D, P, steps, dtype;
  long long Nq;
  size_t sz;
  char* meta = read_file(dir, "meta.txt", &sz);
  if (!meta || sscanf(meta, "%d %d %d %lld %d %d %d", &B, &H, &D, &Nq, &P, &steps, &dtype) != 7) {
    fprintf(stderr, "bad meta.txt\n");
    return 1;
  }
  if (P < 1 || P > DITA_MAX_PARTITIONS || steps < 1 || steps > 64) return 1;
  char* nk_txt = read_file(dir, "nk.txt", &sz);
  int64_t nk[DITA_MAX_PARTITIONS];
  char* cur = nk_txt;
  for (int p = 0; p < P; ++p) nk[p] = strtoll(cur, &cur, 10);
  const size_t esz = dtype == DITA_BF16 ? 2 : 4;
  const size_t o_bytes = (size_t)B * H * Nq * D * esz, l_bytes = (size_t)B * H * Nq * 4;
  dita_shape sh = {B, H, D, dtype, Nq, 0.0f};

  void* q = to_device(read_file(dir, "q.bin", &sz), o_bytes);
  const void* ks[DITA_MAX_PARTITIONS];
  const void* vs[DITA_MAX_PARTITIONS];
  for (int p = 0; p < P; ++p) {
    char name[64];
    const size_t kv_bytes = (size_t)B * H * nk[p] * D * esz;
    snprintf(name, sizeof name, "k%d.bin", p);
    ks[p] = to_device(read_file(dir, name, &sz), kv_bytes);
    snprintf(name, sizeof name, "v%d.bin", p);
    vs[p] = to_device(read_file(dir, name, &sz), kv_bytes);
    if (!ks[p] || !vs[p]) return fail("inputs", DITA_ERR_ARG);
  }
  const size_t cache_bytes = dita_state_cache_bytes(&sh, P);
  void *cache_buf = NULL, *o = NULL, *lse = NULL;
  if (hipMalloc(&cache_buf, cache_bytes) != hipSuccess || hipMalloc(&o, o_bytes) != hipSuccess ||
      hipMalloc(&lse, l_bytes) != hipSuccess || !q)
    return fail("hipMalloc", DITA_ERR_HIP);
  dita_state_cache* cache = NULL;
  int st = dita_state_cache_init(&cache, &sh, P, cache_buf, cache_bytes);
  if (st) return fail("dita_state_cache_init", st);
  void* host_o = malloc(o_bytes);
  void* host_l = malloc(l_bytes);
  for (int s = 0; s < steps; ++s) {
    char name[64];
    snprintf(name, sizeof name, "mask%d.bin", s);
    uint8_t* mask = read_file(dir, name, &sz);
    if (!mask || sz != (size_t)P) return fail("mask", DITA_ERR_ARG);
    dita_step_info info;
    memset(&info, 0, sizeof info);
    st = dita_attn_step(cache, q, ks, vs, nk, mask, s, o, (float*)lse, NULL, &info);
    if (st) return fail("dita_attn_step", st);
    if (hipDeviceSynchronize() != hipSuccess) return fail("sync", DITA_ERR_HIP);
    if (hipMemcpy(host_o, o, o_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(host_l, lse, l_bytes, hipMemcpyDeviceToHost) != hipSuccess)
      return fail("copy back", DITA_ERR_HIP);
    snprintf(name, sizeof name, "o%d.bin", s);
    if (write_file(dir, name, host_o, o_bytes)) return 1;
    snprintf(name, sizeof name, "lse%d.bin", s);
    if (write_file(dir, name, host_l, l_bytes)) return 1;
    char line[64];
    const int len = snprintf(line, sizeof line, "%d %d\n", info.n_fresh, info.n_reused);
    snprintf(name, sizeof name, "info%d.txt", s);
    if (write_file(dir, name, line, (size_t)len)) return 1;
    printf("step %d: fresh %d reused %d\n", s, info.n_fresh, info.n_reused);
    free(mask);
  }
  dita_state_cache_free(cache);
  printf("run ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "check") == 0) return check();
  if (argc >= 3 && strcmp(argv[1], "run") == 0) return run(argv[2]);
  fprintf(stderr, "usage: %s check | run <dir>\n", argv[0]);
  return 2;
}
