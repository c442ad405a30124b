/* Test-session crash reporter (host code only, test infrastructure).
 *
 * On a fatal signal (SIGSEGV, SIGBUS, SIGFPE, SIGILL, SIGABRT) it writes the name of the test that
 * was running and the crashing thread's native stack to stderr, then lets the signal take its
 * default action (the exit status stays that of the signal). Installed before Python's faulthandler,
 * which calls it after its own dump of the Python stacks, so the test name is the last thing the
 * run prints.
 *
 *   gcc -O1 -shared -fPIC crashnote.c -o libcrashnote.so
 */
#define _GNU_SOURCE
#include <execinfo.h>
#include <signal.h>
#include <string.h>
#include <unistd.h>

static char g_note[1024] = "(before the first test)";
static volatile sig_atomic_t g_busy = 0;
static char g_altstack[1 << 16];
static int g_fd = 2; /* a duplicate of stderr taken at install time: a test runner may point fd 2
                        at a capture file while a test runs */

void crashnote_set(const char* s) {
  size_t n = strlen(s);
  if (n >= sizeof g_note) n = sizeof g_note - 1;
  memcpy(g_note, s, n);
  g_note[n] = '\0';
}

static void put(const char* s) {
  ssize_t r = write(g_fd, s, strlen(s));
  (void)r;
}

static void put_int(int v) {
  char buf[16];
  int i = (int)sizeof buf - 1;
  buf[i] = '\0';
  if (v == 0) buf[--i] = '0';
  while (v > 0 && i > 0) {
    buf[--i] = (char)('0' + v % 10);
    v /= 10;
  }
  put(buf + i);
}

static void on_fatal(int sig) {
  if (!g_busy) {
    g_busy = 1;
    put("\n[crashnote] fatal signal ");
    put_int(sig);
    put(" in test ");
    put(g_note);
    put("\n[crashnote] native stack of the crashing thread:\n");
    void* bt[24];
    int n = backtrace(bt, 24);
    backtrace_symbols_fd(bt, n, g_fd);
    put("[crashnote] fatal signal ");
    put_int(sig);
    put(" in test ");
    put(g_note);
    put("\n");
  }
  signal(sig, SIG_DFL);
  raise(sig);
}

int crashnote_install(void) {
  void* warm[2];
  backtrace(warm, 2); /* loads the unwinder now rather than inside the handler */
  const int fd = dup(2);
  if (fd >= 0) g_fd = fd;
  stack_t ss;
  memset(&ss, 0, sizeof ss);
  ss.ss_sp = g_altstack;
  ss.ss_size = sizeof g_altstack;
  sigaltstack(&ss, NULL);
  struct sigaction sa;
  memset(&sa, 0, sizeof sa);
  sa.sa_handler = on_fatal;
  sa.sa_flags = SA_ONSTACK | SA_NODEFER;
  sigemptyset(&sa.sa_mask);
  const int sigs[] = {SIGSEGV, SIGBUS, SIGFPE, SIGILL, SIGABRT};
  for (unsigned k = 0; k < sizeof sigs / sizeof sigs[0]; ++k)
    if (sigaction(sigs[k], &sa, NULL) != 0) return -1;
  return 0;
}
