/* A deliberate heap overflow: the sanitizer test builds this with the same
   flags as the oracle to show that the sanitizer runtime is live (the run
   must abort with a heap-buffer-overflow report). */
#include <stdlib.h>

int main(int argc, char **argv) {
    (void)argv;
    volatile int *a = malloc(4 * sizeof(int));
    int v = a[4 + argc];   /* one past the end and beyond */
    free((void *)a);
    return v == 12345;
}
