/* Plain C99 client of libpfa.so: compiled by the test-suite with gcc against
 * include/pfa.h. It calls only entry points that need no device (version,
 * error strings, argument validation, timing bookkeeping) and prints one line
 * per check; the exit status is the number of failed checks. */
#include <stdio.h>
#include <string.h>

#include "pfa.h"

static int failures = 0;

static void check(int ok, const char* what) {
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    if (!ok) ++failures;
}

int main(void) {
    pfa_shape s;
    int32_t n = -1, dropped = -1;
    char fake_storage[16];
    void* fake = fake_storage; /* never dereferenced: validation fails first */

    check(pfa_version() == 10000, "version 1.0.0");
    check(strcmp(pfa_strerror(PFA_OK), "ok") == 0, "strerror(PFA_OK)");
    check(pfa_strerror(12345) != NULL, "strerror(unknown) not NULL");

    memset(&s, 0, sizeof s);
    s.B = 1; s.heads = 1; s.H = 32; s.W = 32; s.d = 32; s.win = 32; s.shift = 0; s.dtype = PFA_F32;
    check(pfa_sparse_layer(&s, fake, fake, fake, NULL, 0, NULL, 1024, 0, fake, fake, fake, NULL) ==
              PFA_ERR_INVALID, "sparse: K_l = 0 rejected");
    s.d = 8;
    check(pfa_dense_layer(&s, fake, fake, fake, 1024, NULL, NULL, NULL, fake, NULL) == PFA_ERR_UNSUPPORTED,
          "dense: d = 8 unsupported");
    s.d = 32;
    check(pfa_dense_layer(NULL, fake, fake, fake, 1024, NULL, NULL, NULL, fake, NULL) == PFA_ERR_INVALID,
          "dense: NULL shape rejected");
    check(pfa_timing_enable(0) == PFA_OK, "timing off");
    check(pfa_timing_read(NULL, NULL, 0, &n, &dropped) == PFA_OK && n == 0 && dropped == 0, "timing read empty");
    check(strcmp(pfa_kernel_name(PFA_KERNEL_DENSE), "dense_layer_kernel") == 0, "kernel family name");
    return failures;
}
